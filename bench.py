"""Benchmark of the decode-step MoE FFN on one MI355X.

One step = one pass of the whole layer (routing, grouping when rows >= 2,
gate/up + silu*mul, down + blend into the residual) over every resident
layer of the workload, back to back on one stream, inputs already in HBM.
Default workload: the 35B-A3B shape at one decode row (hidden 2048, 256
experts top-8, intermediate 512, a gated shared expert, fp8 e4m3 block-128
weights), 40 independent layers so the touched weights (~1.17 GB per step)
exceed the on-package cache.

Prints one JSON line (rank 0).  value = effective weight GB/s (each distinct
touched expert's codes and scales once per step, the shared expert, the
shared-gate vector and the router matrix) over the timed steps; us_per_layer
and pct_hbm_peak are given beside it.  `roofline` is for the dominant kernel,
timed with HIP events on the launch stream; `cpu_baseline` is the CPU oracle
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FMT_DTYPE = {0: "fp8e4m3", 1: "nvfp4", 2: "int8", 3: "int4", 4: "int4", 5: "fp8e4m3"}
FMT_NAME = {0: "fp8 e4m3 block-128", 1: "nvfp4", 2: "int8 per-row", 3: "int4 per-row", 4: "int4-g64",
            5: "fp8 e4m3 block-128, bf16 scales"}
METRIC = "us per MoE layer + effective weight GB/s (% of HBM peak), 35B-A3B shape, n=1"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="a3b")
    p.add_argument("--rows", type=int, default=None)
    p.add_argument("--layers", type=int, default=None)
    p.add_argument("--launch", choices=["graph", "stream", "both"], default="both")
    p.add_argument("--norm", action="store_true",
                   help="with the RMSNorm epilogue of the layer output (moe_layer_forward_norm)")
    p.add_argument("--dense", default=None, metavar="SHAPE",
                   help="time the dense fp8 block-128 projection (moe_dense_fp8) of this shape instead")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--profile-steps", type=int, default=None,
                   help="run exactly this many steps (no warmup, no report) for profilers")
    p.add_argument("--phases", type=int, default=None, metavar="N",
                   help="phase stamps of N one-launch layers (cycling the resident layers, a sync between "
                        "calls) instead of the timing: when each workgroup role reaches each phase")
    p.add_argument("--copy-calibration", type=int, default=None, metavar="MIB",
                   help="run 10 device-to-device copies of MIB MiB (the counter calibration kernel)")
    return p.parse_args()


def distinct_routed(res) -> int:
    """Distinct routed experts touched per step, summed over layers."""
    import torch
    total = 0
    for rt in res.routing:
        total += int(torch.unique(rt.topk_ids).numel())
    return total


CSRC = os.path.join(ROOT, "routed_fp8_expert_amd", "csrc")
# translation unit of each profiled kernel
KERNEL_TU = {"layer": "layer.hip", "dense": "dense.hip"}


def _digest(names) -> str:
    h = hashlib.sha256()
    for name in sorted(names):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def source_digest(kernel: str = None) -> str:
    """Digest of the native sources: all of them, or those a kernel's code
    depends on (its translation unit, the headers it includes, directly or
    not, and the C ABI's host code that sizes and launches it)."""
    if kernel is None:
        return _digest(os.listdir(CSRC))
    names, todo = set(), [KERNEL_TU[kernel], "api.cpp", "host_checks.hpp"]
    while todo:
        name = todo.pop()
        if name in names or not os.path.exists(os.path.join(CSRC, name)):
            continue
        names.add(name)
        with open(os.path.join(CSRC, name)) as f:
            todo += re.findall(r'^\s*#\s*include\s+"([^"]+)"', f.read(), re.M)
    return _digest(names)


def counter_traffic(kernel: str, workload: str, rows: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this kernel and workload (profiles/traffic_<kernel>_<workload>_r<rows>.txt,
    `key: value` lines), if it was taken on the current sources of that
    kernel."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}_r{rows}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith((" ", "#")):
                key, _, val = line.partition(":")
                kv[key.strip()] = val.strip()
    if kv.get("source_digest") != source_digest(kernel):
        return None
    return int(kv["hbm_bytes_per_launch"]) if "hbm_bytes_per_launch" in kv else None


def cpu_threads():
    """Threads the oracle may use: every CPU of this process's affinity mask,
    capped by OMP_NUM_THREADS where the environment sets it (a shared GPU machine
    grants each GPU a share of its CPUs that way)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_info() -> dict:
    """Seed, sources and software versions of the run."""
    import subprocess
    import torch
    import moe_synth as syn
    rev = None
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        rev = r.stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        pass
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"seed": syn.BASE_SEED, "git_revision": rev, "source_digest": source_digest(), "rocm": rocm,
            "hip_runtime": torch.version.hip, "torch": torch.__version__,
            "gpu": torch.cuda.get_device_name(0) if torch.cuda.is_available() else None}


def verify_layer(moe, oracle, L, wl, res, ctx, stream, n, x, li, logits):
    """Layer n once more on the GPU with y written (a fresh copy of its
    residual; outside the timed region), checked against the oracle layer L:
    ids bit-exact, weights within 1e-5, y within max|err| <= 2e-2 * rms(y)
    and sum|err| / sum|y| <= 5e-3.  A layer whose oracle logits put two of the
    k+1 largest within 1e-4 of each other (where a different summation order
    may legitimately swap them) is reported as a near tie, not compared."""
    import numpy as np
    import torch
    from oracle.layers import bits, min_top_gap
    gap = min_top_gap(logits, wl.top_k)
    if gap < 1e-4:
        return {"layer": res.layer_ids[n], "near_tie": round(gap, 8)}
    ref = oracle.layer_forward(L, x, logits_in=li, residual=bits(res.residual0[n]))
    rows = res.rows
    y = torch.empty((rows, wl.hidden), dtype=torch.bfloat16, device=res.device)
    rt = moe.Routing(rows, wl.n_experts, wl.top_k, res.device)
    resid = res.residual0[n].clone()
    moe.moe_layer_forward(ctx, res.lw[n], res.x[n], y, resid, res.ws, logits_in=res.logits_in[n],
                          routing=rt, stream=stream)
    torch.cuda.synchronize()
    ids_ok = bool(np.array_equal(rt.topk_ids.cpu().numpy(), ref["ids"]))
    w_err = float(np.max(np.abs(rt.topk_w.cpu().numpy() - ref["w"])))
    g = y.float().cpu().numpy().astype(np.float64)
    o = ref["y"].astype(np.float64)
    rms = float(np.sqrt(np.mean(o * o)))
    err = np.abs(g - o)
    max_rel = float(err.max() / max(rms, 1e-300))
    mean_rel = float(err.sum() / max(np.abs(o).sum(), 1e-300))
    ok = ids_ok and w_err <= 1e-5 and max_rel <= 2e-2 and mean_rel <= 5e-3 and bool(np.all(np.isfinite(g)))
    return {"layer": res.layer_ids[n], "ok": ok, "ids_equal": ids_ok, "w_max_err": w_err,
            "y_max_err_over_rms": max_rel, "y_mean_rel_err": mean_rel}


def cpu_baseline(wl, res, budget_s: float, moe, ctx, stream):
    """The CPU oracle on the same layers (touched experts copied to the host
    outside the timing), layer by layer until the time budget is spent; each
    layer it runs is also the parity check of that layer's GPU result
    (verify_layer)."""
    import numpy as np
    import oracle
    from oracle.layers import bits, host, oracle_layer, router_only_layer
    import moe_synth as syn

    threads = cpu_threads()
    oracle.set_threads(threads)
    done_layers, t_total, bytes_total = 0, 0.0, 0
    checks = []
    for n in range(len(res.layer_ids)):
        x = bits(res.x[n])
        li = host(res.logits_in[n])
        logits = li if li is not None else oracle.router_logits(router_only_layer(oracle, wl, res.W[n]), x)
        ids_orc, _ = oracle.topk_softmax(logits, wl.top_k)
        ids_gpu = res.routing[n].topk_ids.cpu().numpy()
        # touched experts to the host (outside the timing): the oracle's own
        # choice, and the GPU's (they differ only on a near tie)
        L = oracle_layer(oracle, wl, res.W[n], experts=np.union1d(ids_orc, ids_gpu))
        t0 = time.perf_counter()
        oracle.layer_forward(L, x, logits_in=li)
        t_total += time.perf_counter() - t0
        done_layers += 1
        bytes_total += syn.effective_weight_bytes(wl, int(np.unique(ids_orc).size), li is None)
        checks.append(verify_layer(moe, oracle, L, wl, res, ctx, stream, n, x, li, logits))
        if n == 0:
            first = (L, x, li)
        if t_total >= budget_s:
            break
    # the first layer again on one thread
    oracle.set_threads(1)
    L, x, li = first
    t0 = time.perf_counter()
    oracle.layer_forward(L, x, logits_in=li)
    t_one = time.perf_counter() - t0
    oracle.set_threads(threads)
    compared = [c for c in checks if "ok" in c]
    parity = {
        "layers_compared": len(compared),
        "layers_near_tie": len(checks) - len(compared),
        "ok": all(c["ok"] for c in compared) and len(compared) > 0,
        "worst_y_max_err_over_rms": max((c.get("y_max_err_over_rms", 0.0) for c in compared), default=None),
        "worst_y_mean_rel_err": max((c.get("y_mean_rel_err", 0.0) for c in compared), default=None),
        "failed": [c for c in compared if not c["ok"]][:4],
    }
    cpu = {
        "value": round(bytes_total / t_total / 1e9, 4),
        "unit": "GB/s",
        "us_per_layer": round(t_total / done_layers * 1e6, 1),
        "cores": threads,
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{done_layers} of {len(res.layer_ids)} layers of the same workload, one pass each, "
                  f"{threads} OpenMP threads, f64 arithmetic; layer 0 once more on 1 thread",
        "single_thread_us_per_layer": round(t_one * 1e6, 1),
    }
    return cpu, parity


PHASES = {
    0: ["start", "row dot done", "done words stored"],
    1: ["start", "-", "-", "h stored", "done words stored"],
    2: ["start", "routing done words seen", "top-k done", "h stored", "done words stored", "-", "-", "-", "-",
        "logits arrived"],
    3: ["start", "routing done words seen", "top-k done", "down-row loads issued", "gate/up done words seen",
        "h staged", "blend stored", "group arrival returned", "group line cleared (last of its group)",
        "logits arrived"],
}
# table order of the phases per role (stamp word numbers)
PHASE_ORDER = {0: [1, 2, 3], 1: [1, 4, 5], 2: [1, 2, 10, 3, 4, 5], 3: [1, 2, 10, 3, 4, 5, 6, 7, 8, 9]}
ROLES = {0: "router", 1: "shared gate/up", 2: "routed gate/up", 3: "down"}


def run_phases(args, wl, res, moe, ctx, stream, layers):
    """Phase stamps of the one-launch layer: per call, each workgroup's
    constant-clock stamps relative to the earliest workgroup start of that
    call; per role and phase the median and the latest workgroup, averaged
    over the calls.  Also the back-to-back time per layer of the same
    workload (no stamps) for the launch boundary."""
    import numpy as np
    import torch

    def step():
        res.run(ctx, stream=stream, write_y=False)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    with torch.cuda.stream(stream):
        ev[0].record(stream)
        for _ in range(args.steps):
            step()
        ev[1].record(stream)
    torch.cuda.synchronize()
    us_layer = ev[0].elapsed_time(ev[1]) * 1e3 / args.steps / layers
    buf = torch.full((8192 * 16,), -1, dtype=torch.int64, device=res.device)
    khz = moe.moe_debug_set_phase_stamps(ctx, buf)
    per_us = khz / 1000.0
    med = {}
    mx = {}
    spans = []
    for i in range(args.phases):
        n = i % layers
        buf.fill_(-1)
        torch.cuda.synchronize()
        moe.moe_layer_forward(ctx, res.lw[n], res.x[n], None, res.residual[n], res.ws,
                              logits_in=res.logits_in[n], routing=res.routing[n], stream=stream)
        torch.cuda.synchronize()
        w = buf.view(-1, 16).cpu().numpy()
        w = w[w[:, 1] >= 0]
        t0 = w[:, 1].min()
        role = w[:, 0] & 0xFF
        spans.append((w[:, 1:][w[:, 1:] >= 0].max() - t0) / per_us)
        for r in PHASES:
            sel = w[role == r]
            for j in range(1, len(PHASES[r]) + 1):
                v = sel[:, j]
                v = v[v >= 0]
                if v.size == 0:
                    continue
                t = (v - t0) / per_us
                med.setdefault((r, j), []).append(float(np.median(t)))
                mx.setdefault((r, j), []).append(float(t.max()))
    moe.moe_debug_set_phase_stamps(ctx, None)
    assert moe.moe_ctx_device_errors(ctx, clear=False) == 0
    print(f"| role | phase | median workgroup (us) | latest workgroup (us) |")
    print("|---|---|---|---|")
    for r in PHASES:
        for j in PHASE_ORDER[r]:
            if (r, j) in med:
                print(f"| {ROLES[r]} | {PHASES[r][j - 1]} | {np.mean(med[(r, j)]):.2f} | {np.mean(mx[(r, j)]):.2f} |")
    span = float(np.mean(spans))
    print()
    print(f"calls: {args.phases} (layers cycled, a synchronisation between calls); constant clock {khz} kHz")
    print(f"first workgroup start to last stamp: {span:.2f} us (mean over calls)")
    print(f"back to back without stamps ({args.steps} steps x {layers} layers): {us_layer:.2f} us per layer; "
          f"the difference, {us_layer - span:.2f} us, is the launch boundary, the dispatch ramp before the "
          f"first start and the tail after the last stamp")


def run_dense(args):
    """The dense fp8 block-128 projection: `copies` resident matrices of one
    shape (together beyond the on-package cache) applied in turn to the same
    rows; one step = one projection per copy."""
    import numpy as np
    import torch
    import moe_synth as syn
    import routed_fp8_expert_amd as moe

    name = args.dense
    n, k = syn.DENSE_SHAPES[name]
    rows = args.rows if args.rows is not None else 1
    wbytes = n * k + (n // 128) * (k // 128) * 4
    copies = args.layers if args.layers is not None else max(8, -(-(1 << 30) // wbytes))
    torch.cuda.set_device(0)
    q, s = syn.make_dense_weights(name, n, k, "cuda")
    mats = []
    for c in range(copies):
        qc, sc = q.clone(), s.clone()
        mats.append((qc, sc, moe.DenseWeights(qc, sc)))
    x = syn.make_dense_x(name, rows, k, "cuda")
    y = torch.empty((rows, n), dtype=torch.bfloat16, device="cuda")
    ctx = moe.Ctx(0)
    stream = torch.cuda.Stream()

    def step():
        for _, _, w in mats:
            moe.moe_dense_fp8(ctx, w, x, y, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    with torch.cuda.stream(stream):
        ev[0].record(stream)
        for _ in range(args.steps):
            step()
        ev[1].record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev[0].elapsed_time(ev[1]) / args.steps
    us = ms_per_step * 1e3 / copies
    assert moe.moe_ctx_status(ctx) == 0

    moe.moe_ctx_set_timing(ctx, True)
    kt_steps = min(args.steps, 20)
    for _ in range(kt_steps):
        step()
    torch.cuda.synchronize()
    kms, kn = moe.moe_ctx_kernel_stats(ctx, moe.KERNELS.index("dense"))
    moe.moe_ctx_set_timing(ctx, False)
    ctx.close()
    # algorithmic bytes per launch: codes + scales once, x read, y written
    alg = wbytes + rows * k * 2 + rows * n * 2
    flops = 2.0 * rows * n * k
    achieved = alg / (us * 1e-6) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = cpu_threads()
        oracle.set_threads(threads)
        qh, sh = q.cpu().numpy(), s.cpu().numpy()
        xb = x.cpu().view(torch.int16).numpy().view(np.uint16)
        t0, done = time.perf_counter(), 0
        while time.perf_counter() - t0 < args.cpu_seconds:
            oracle.dense_fp8(qh, sh, xb)
            done += 1
        t = (time.perf_counter() - t0) / done
        cpu = {"value": round(alg / t / 1e9, 4), "unit": "GB/s", "us_per_projection": round(t * 1e6, 1),
               "cores": threads, "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
               "kind": "oracle",
               "sample": f"{done} projections of the same shape and rows, {threads} OpenMP threads, f64"}
    line = {
        "metric": f"us per dense fp8 block-128 projection {n}x{k} + weight GB/s (% of HBM peak), {rows} row(s)",
        "value": round(achieved, 1),
        "unit": "GB/s",
        "us_per_projection": round(us, 3),
        "pct_hbm_peak": round(100.0 * achieved / HBM_PEAK_GBS, 2),
        "tflops": round(flops / (us * 1e-6) / 1e12, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3-w/bf16-x/f32-acc",
        "data": "synthetic (seeded; weights N(0,0.02) quantised, activations N(0,1))",
        "config": {"workload": f"dense {name}: y[{rows},{n}] = x[{rows},{k}] . W^T, fp8 e4m3 block-128 weights, "
                               f"{copies} resident copies in turn",
                   "rows": rows, "copies": copies,
                   "arm": "matrix cores" if rows >= 8 else "gemv"},
        "kernels": {"dense": {"avg_us": round(kms / max(kn, 1) * 1e3, 3), "launches_per_step": kn // kt_steps}},
        "roofline": {"bound": "hbm", "kernel": "dense", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic("dense", name, rows),
                     "algorithmic_bytes_per_launch": int(alg)},
        "cpu_baseline": cpu,
        "source_digest": source_digest(),
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    if args.copy_calibration is not None:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        torch.cuda.synchronize()
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 10}))
        return

    if args.dense is not None:
        run_dense(args)
        return

    import moe_synth as syn
    import routed_fp8_expert_amd as moe
    from routed_fp8_expert_amd.workload import Resident

    wl = syn.WORKLOADS[args.workload]
    rows = args.rows if args.rows is not None else wl.rows[0]
    layers = args.layers if args.layers is not None else wl.layers
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    progress = None
    if args.profile_steps is not None:
        def progress(msg):
            print(msg, file=sys.stderr, flush=True)
    res = Resident(wl, rows, layers, device=dev, keep_y=False, norm=args.norm, progress=progress)
    ctx = moe.Ctx(0)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    if args.phases is not None:
        run_phases(args, wl, res, moe, ctx, stream, layers)
        ctx.close()
        return

    def step():
        res.run(ctx, stream=stream, write_y=False)

    if args.profile_steps is not None:
        with torch.cuda.stream(stream):
            for i in range(args.profile_steps):
                step()
                torch.cuda.synchronize()
                print(f"profiled step {i + 1} of {args.profile_steps}", file=sys.stderr, flush=True)
        errors = moe.moe_ctx_device_errors(ctx, clear=False)
        print(json.dumps({"profile_steps": args.profile_steps, "workload": wl.name, "rows": rows,
                          "device_errors": errors}))
        ctx.close()
        if errors:
            sys.exit(1)
        return

    results = {}
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()

    # An event after every step on the launch stream: the timed region is
    # first..last event, and the per-step spans give the distribution.
    def timed(run_one):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            ev[0].record(stream)
            for i in range(args.steps):
                run_one()
                ev[i + 1].record(stream)
        torch.cuda.synchronize()
        spans = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
        return ev[0].elapsed_time(ev[-1]) / args.steps, spans

    def time_graph():
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            step()
        torch.cuda.synchronize()
        for _ in range(max(3, args.warmup // 4)):
            g.replay()
        torch.cuda.synchronize()
        return timed(g.replay)

    spans_by_mode = {}
    if args.launch in ("stream", "both"):
        results["stream"], spans_by_mode["stream"] = timed(step)
    if args.launch in ("graph", "both"):
        results["graph"], spans_by_mode["graph"] = time_graph()
    assert moe.moe_ctx_status(ctx) == 0
    device_errors = moe.moe_ctx_device_errors(ctx, clear=False)
    best_mode = min(results, key=results.get)
    ms_per_step = results[best_mode]

    def pct(v, q):
        v = sorted(v)
        return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]
    spans = spans_by_mode[best_mode]
    dist = {f"p{q}": round(pct(spans, q / 100) * 1e3 / layers, 3) for q in (10, 50, 90)}

    # rows per expert over the step (multi-row steps): the grouping's counts
    routing_stats = None
    if rows >= 2:
        cnt = torch.stack([torch.bincount(rt.topk_ids.flatten().to(torch.int64), minlength=wl.n_experts)
                           for rt in res.routing])   # [layers, E]
        routing_stats = {
            "distinct_experts_per_layer": round(float((cnt > 0).sum(1).float().mean()), 2),
            "zero_row_experts_per_layer": round(float((cnt == 0).sum(1).float().mean()), 2),
            "max_rows_per_expert": int(cnt.max()),
            "experts_ge_4_rows_per_layer": round(float((cnt >= 4).sum(1).float().mean()), 2),
            "experts_ge_32_rows_per_layer": round(float((cnt >= 32).sum(1).float().mean()), 2),
            "row_histogram_layer0": {str(int(b)): int(n) for b, n in
                                     zip(*torch.unique(cnt[0], return_counts=True))},
        }
    router_gemv = wl.router == "gemv"
    eff_bytes = sum(syn.effective_weight_bytes(wl, int(torch.unique(rt.topk_ids).numel()), router_gemv)
                    for rt in res.routing)
    gbs = eff_bytes / (ms_per_step * 1e-3) / 1e9
    us_layer = ms_per_step * 1e3 / layers

    # per-kernel durations with HIP events around each launch (separate pass)
    moe.moe_ctx_set_timing(ctx, True)
    kt_steps = min(args.steps, 50)
    for _ in range(kt_steps):
        step()
    torch.cuda.synchronize()
    kernels = {}
    for kid, name in enumerate(moe.KERNELS):
        ms, n = moe.moe_ctx_kernel_stats(ctx, kid)
        if n:
            kernels[name] = {"avg_us": round(ms / n * 1e3, 3), "launches_per_step": n // kt_steps}
    moe.moe_ctx_set_timing(ctx, False)
    device_errors |= moe.moe_ctx_device_errors(ctx, clear=False)

    # Algorithmic bytes of one layer: the effective weight bytes plus the
    # activations read (x) and the residual read and written.
    H, E, I, Is, k = wl.hidden, wl.n_experts, wl.inter, wl.shared_inter, wl.top_k
    act_bytes = rows * H * 2 + 2 * rows * H * 2
    layer_bytes = eff_bytes / layers + act_bytes
    roofline = None
    if "layer" in kernels:
        # One kernel per layer: it is the dominant (and only) kernel, and its
        # average launch duration is the timed region (HIP events on the
        # launch stream) over the launches in it; the per-launch event pairs
        # of the diagnostic pass add their own overhead and are reported aside.
        kernels["layer"]["avg_us_timed_region"] = round(us_layer, 3)
        achieved = layer_bytes / (us_layer * 1e-6) / 1e9
        traffic = counter_traffic("layer", wl.name, rows)
        roofline = {"bound": "hbm", "kernel": "layer", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "algorithmic_bytes_per_launch": int(layer_bytes)}
    elif kernels:
        # several kernels per layer: the layer's bytes over the sum of its kernels' times
        us = sum(st["avg_us"] * st["launches_per_step"] for st in kernels.values()) / layers
        achieved = layer_bytes / (us * 1e-6) / 1e9
        dominant = max(kernels, key=lambda n: kernels[n]["avg_us"] * kernels[n]["launches_per_step"])
        roofline = {"bound": "hbm", "kernel": "all kernels of a layer (dominant: %s)" % dominant,
                    "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                    "algorithmic_bytes_per_launch": int(layer_bytes)}

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(wl, res, args.cpu_seconds, moe, ctx, stream)
        device_errors |= moe.moe_ctx_device_errors(ctx, clear=False)

    line = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "us_per_layer": round(us_layer, 3),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_layer_dist": dist,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": FMT_DTYPE[wl.fmt] + "-w/bf16-x/f32-acc",
        "data": "synthetic (seeded; weights N(0,0.02) quantised, activations N(0,1) RMS-normalised)",
        "config": {"workload": f"{wl.name}: hidden {H}, {E} experts top-{k}, inter {I}, shared inter {Is}, "
                               f"{FMT_NAME[wl.fmt]} weights, "
                               f"{rows} row(s), {layers} layers back to back",
                   "rows": rows, "layers": layers, "launch": best_mode,
                   "router": wl.router, "epilogue": "rmsnorm" if args.norm else None},
        "launch_ms_per_step": {m: round(v, 5) for m, v in results.items()},
        "effective_bytes_per_step": int(eff_bytes),
        "routing": routing_stats,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "device_errors": device_errors,
        "run": run_info(),
    }
    ctx.close()
    if device_errors or (parity is not None and not parity["ok"]):
        # a timed run whose kernels flagged an error, or whose checked layers
        # differ from the oracle, measured something other than the layer
        print(json.dumps({"error": "the timed layers are not valid: "
                          + (f"device error word {device_errors:#x}" if device_errors else "parity check failed"),
                          "metric": METRIC, "device_errors": device_errors, "parity": parity,
                          "config": line["config"], "run": line["run"]}), flush=True)
        sys.exit(1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
