"""Throughput of the Muon update on one MI355X, GPT-2-124M hidden-matrix set.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                [--no-cpu-baseline] [--cpu-budget SECONDS] [--calibrate-copy]
                [--vendor-ceiling]

A step is one muon_plan_step over all matrices of the workload (momentum,
normalisation and k Newton-Schulz steps), inputs resident in HBM, one plan
over fixed gradient buffers as in training (the momentum buffers evolve from
step to step). `step_ms` gives the spread of single steps from a separate
pass with events around each step. `value` is
algorithmic TFLOP/s of the whole step; `roofline` describes the kernel with
the largest share of the step's time against its matrix-core roof (HBM under
`roofline.other`), timed with HIP events recorded around
each launch in a second pass of the same length (in that pass the launches
run one at a time on the step's stream, so each interval holds one launch;
the timed pass runs the Newton-Schulz steps as one chained launch where the
plan has one, else as separate launches with large sets in concurrent
groups; `separate_launches_ms_per_step` times the latter for comparison); the
CPU baseline times the float64 oracle on a bounded sample of the same
matrices. `roofline.traffic` is the dominant kernel's HBM bytes per launch
from the committed rocprofv3 counter summary (null if that summary was taken
on a different kernel source). Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Muon NS orthogonalisation TFLOPS & % bf16 MFMA peak, GPT-2-124M matrix set"
PEAK = {"bf16": 2500.0, "fp32": 157.3}       # dense MFMA TFLOP/s, MI355X
HBM_PEAK_GBS = 8000.0


def kernel_work(shapes, steps, dtype):
    """Algorithmic work of each kernel per update step (all its launches):
    {kernel: (flops, bytes)}.

    Bytes count each operand read once and each result written once, in the
    library's formats: bf16 sets (fp16 operands) keep X as a 16-bit high part
    (the matrix-core operand) and a one-byte low part (the residual), and A, B
    as 16-bit; fp32 sets keep everything in fp32. With at least one step,
    bf16 sets write X0 (scaled by a power of two: high part and low byte) in
    the momentum pass, and the normalise slot only reduces per-tile sums (no
    matrix bytes; its rewrites, when the plan's guess of X0's power of two
    was wrong, are not algorithmic work). The Newton-Schulz kernels run
    `steps` times; the last update writes `out` instead of X's parts. `chain`
    (the chained launch) is the Gram, poly and update work together."""
    es = 2 if dtype == "bf16" else 4
    xb = 3 if dtype == "bf16" else 4        # X per element: hi + lo byte, or fp32
    xop = 2 if dtype == "bf16" else 4       # X as a matrix-core operand (high half)
    fused = dtype == "bf16" and steps > 0
    w = {k: [0.0, 0.0] for k in ("momentum", "normalize", "gram", "poly", "update")}
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        mn, mm = float(m * n), float(m * m)
        if fused:
            w["momentum"][1] += 3 * es * mn + xb * mn    # read G, buf; write buf', X0
        else:
            w["momentum"][1] += 3 * es * mn              # read G, buf; write buf'
            w["normalize"][1] += 2 * es * mn + xb * mn   # read G, buf'; write X
        w["gram"][0] += steps * m * (m + 1) * n
        w["gram"][1] += steps * (xop * mn + es * mm)       # read X operand; write A
        w["poly"][0] += steps * m * m * (m + 1)
        w["poly"][1] += steps * 2 * es * mm                # read A; write B
        w["update"][0] += steps * 2 * m * m * n
        for t in range(steps):
            out = es if t == steps - 1 else xb                             # write out, or X
            w["update"][1] += es * mm + xb * mn + out * mn                 # read B, X
    w["chain"] = [w["gram"][0] + w["poly"][0] + w["update"][0], w["gram"][1] + w["poly"][1] + w["update"][1]]
    return {k: (v[0], v[1]) for k, v in w.items()}


def roofline_of(flops, nbytes, secs, dtype):
    """Roofline entry of a matrix-core kernel's work in `secs`: the headline
    is the matrix-core roof (algorithmic flops over the dense MFMA peak of
    the operand type: fp16 and bf16 share 2.5 PFLOP/s on MI355X); the HBM
    figure (algorithmic bytes over 8 TB/s) is kept under `other`, with both
    lower bounds on the time."""
    mf = {"bound": "mfma", "achieved": flops / secs / 1e12, "peak": PEAK[dtype],
          "unit": "TFLOP/s"}
    hb = {"bound": "hbm", "achieved": nbytes / secs / 1e9, "peak": HBM_PEAK_GBS,
          "unit": "GB/s"}
    for r in (mf, hb):
        r["frac"] = r["achieved"] / r["peak"]
    mf["other"] = hb
    mf["bound_us"] = {"hbm": nbytes / (HBM_PEAK_GBS * 1e9) * 1e6,
                      "mfma": flops / (PEAK[dtype] * 1e12) * 1e6}
    return mf


def vendor_ceiling(wl, reps: int = 50):
    """Empirical ceiling from the vendor GEMM (hipBLASLt through torch,
    bf16 operands, fp32 accumulation): dense TFLOP/s of batched GEMMs at the
    step's shapes (one launch per shape group) and of one 8192^3 GEMM, and a
    plain torch version of the whole
    Newton-Schulz part of the step (batched products over each shape group,
    every operand contiguous), timed with events on the current stream."""
    import torch
    dev = torch.device("cuda:0")
    torch.manual_seed(0)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    # batched over a shape group, so that one launch fills the GPU (single
    # small GEMMs measure the host's launch rate, not the matrix cores)
    gemms = {}
    for (bt, m, k, n) in [(48, 768, 768, 768), (24, 768, 3072, 768), (24, 768, 768, 3072),
                          (96, 1024, 1024, 1024), (24, 1024, 4096, 1024), (24, 1024, 1024, 4096),
                          (32, 2048, 8192, 2048), (32, 2048, 2048, 8192), (1, 8192, 8192, 8192)]:
        x = torch.randn(bt, m, k, device=dev, dtype=torch.bfloat16)
        y = torch.randn(bt, k, n, device=dev, dtype=torch.bfloat16)
        t = timed(lambda: torch.bmm(x, y))
        gemms[f"{bt}x({m}x{k}x{n})"] = {"us": t * 1e6, "TFLOP/s": 2.0 * bt * m * k * n / t / 1e12}
        del x, y
    # the step's Newton-Schulz part in plain torch (X in rows <= cols form)
    groups = {}
    for r, c in wl.shapes:
        groups[(min(r, c), max(r, c))] = groups.get((min(r, c), max(r, c)), 0) + 1
    xs = [torch.randn(cnt, m, n, device=dev, dtype=torch.bfloat16) / (m * n) ** 0.5
          for (m, n), cnt in groups.items()]
    a, b, c = wl.coeffs

    def ns():
        for x in xs:
            y = x
            for _ in range(wl.steps):
                A = torch.bmm(y, y.transpose(1, 2).contiguous())
                B = b * A + c * torch.bmm(A, A)
                y = a * y + torch.bmm(B, y)
    t = timed(ns)
    return {"gemm": gemms,
            "torch_ns_step": {"ms": t * 1e3, "TFLOP/s_alg": wl.falg_flops() / t / 1e12,
                              "note": "Newton-Schulz part only (no momentum or normalisation), "
                                      "bf16 torch.bmm per shape group, k steps"}}


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per update step of `kernel` (all its launches) from the
    committed rocprofv3 counter summary (FETCH_SIZE / WRITE_SIZE scaled by a
    plain-copy calibration), or None when it is missing or was taken on a
    different kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    src = os.path.join(ROOT, "muon_newton_schulz_04_amd", "csrc", "kernels.hip")
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(src, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if rec.get("kernel_source_sha256") != sha:
        return None
    ent = rec.get("per_step", {}).get(kernel)
    return None if ent is None else ent["traffic_bytes"]


def cpu_baseline(wl, budget_s: float = 12.0):
    """Float64 oracle on the host cores over whole layers of the workload
    (one layer = 4 square + 1 wide + 1 tall matrix), cycling through the
    layers until at least budget_s of oracle time has accumulated."""
    import oracle
    from threadpoolctl import threadpool_info
    from workloads import make_gradients, to_f64

    L = wl.n_matrices // 6 if wl.n_matrices % 6 == 0 else 0
    layer_idx = (lambda l: [4 * l, 4 * l + 1, 4 * l + 2, 4 * l + 3, 4 * L + l, 5 * L + l]) \
        if L else (lambda l: [l])
    nlayers = L if L else wl.n_matrices
    grads = make_gradients(wl, step=0, device="cpu")
    done, flops, t_total = 0, 0, 0.0
    a, b, c = (float(np.float32(x)) for x in wl.coeffs)
    while t_total < budget_s:
        idx = layer_idx(done % nlayers)
        g64 = [to_f64(grads[i]) for i in idx]
        t0 = time.perf_counter()
        for g in g64:
            oracle.muon_update(g, np.zeros_like(g), a=a, b=b, c=c, steps=wl.steps,
                               mu=float(np.float32(wl.momentum)), nesterov=wl.nesterov,
                               eps=wl.eps, buf_dtype=wl.dtype)
        t_total += time.perf_counter() - t0
        flops += sum(oracle.falg_flops(*wl.shapes[i], wl.steps) for i in idx)
        done += 1
    threads = max([p.get("num_threads", 1) for p in threadpool_info()
                   if p.get("user_api") == "blas"] or [1])
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} {'layers (6 matrices each)' if L else 'matrices'} "
                      f"({done / nlayers:.2f} passes over the {wl.n_matrices} matrices) of "
                      f"{wl.name}, float64 NumPy, {t_total:.1f} s",
            "seconds": t_total, "host_cpus": os.cpu_count()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 30 warm-up steps: after an idle pause the first step runs at the idle
    # clock, the next ones at a clock the power controller has pulled far
    # down, and the step time settles over about 20 to 30 steps (measured on
    # the GPT-2-124M set: 1.52 ms, then 2.2 ms, falling to 1.60 ms)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="gpt2_124m_matrix_set")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--vendor-ceiling", action="store_true",
                    help="only time the vendor GEMM (hipBLASLt via torch) at the workload's "
                         "shapes and a plain torch Newton-Schulz step, then exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 512 MiB three times (the "
                         "reference for scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        src = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": src.numel(), "copies": 3}))
        return
    if args.vendor_ceiling:
        from workloads import CONFIGS
        print(json.dumps({"vendor_ceiling": vendor_ceiling(CONFIGS[args.workload]),
                          "workload": args.workload}), flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} / WORLD_SIZE {world} "
              "is not supported (a several-GPU step would give each rank whole matrices to "
              "update; only one rank's share is timed, under next.rank_share).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import muon_newton_schulz_04_amd as mu
    from workloads import CONFIGS, make_gradients

    wl = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # one plan over fixed gradient buffers, as in training (backward rewrites
    # the same .grad tensors every step); the momentum buffers evolve
    # (sets beyond 2^28 elements are generated on the GPU: the host's QR
    # factorisations of the power-law set take minutes)
    gen_dev = "cuda" if sum(r * c for r, c in wl.shapes) > (1 << 28) else "cpu"
    print(f"bench: generating {wl.n_matrices} matrices of {wl.name} on {gen_dev}", file=sys.stderr, flush=True)
    grads = [g.to(dev) for g in make_gradients(wl, step=0, device=gen_dev)]
    print("bench: inputs ready", file=sys.stderr, flush=True)
    bufs = [torch.zeros_like(g) for g in grads] if wl.momentum else None
    outs = [torch.empty_like(g) for g in grads]
    plan = mu.MuonPlan(grads, bufs, outs)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    cfg = mu.make_config(*wl.coeffs, wl.steps, wl.momentum, wl.nesterov, wl.eps)
    stream = torch.cuda.current_stream()

    for i in range(args.warmup):
        plan.step(cfg, ws, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        plan.step(cfg, ws, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps

    # spread of single steps: a pass of the same length with events around
    # every step (outside the timed region above)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for i, (a0, a1) in enumerate(ev):
        a0.record(stream)
        plan.step(cfg, ws, stream)
        a1.record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([a0.elapsed_time(a1) for a0, a1 in ev])

    # the same step captured once as a HIP graph (the step allocates nothing
    # and issues no memset, so it is capture-safe) and replayed
    # (a capture that fails is reported in the line, not fatal)
    try:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            plan.step(cfg, ws)
        torch.cuda.synchronize()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        hip_graph = {"ms_per_step": e0.elapsed_time(e1) / args.steps, "steps": args.steps,
                     "note": "one muon_plan_step captured once and replayed; value is the eager rate"}
        del graph
    except RuntimeError as exc:
        torch.cuda.synchronize()
        hip_graph = {"error": str(exc)[:200]}

    # the step form the timed pass used (the chained launch where the plan
    # has one), and the same step with the separate launches (three per
    # Newton-Schulz step, large sets as concurrent groups) for comparison
    chained, chain_err = plan.chain_state()
    separate = None
    if chained:
        plan.set_chained(False)
        e0.record(stream)
        for _ in range(args.steps):
            plan.step(cfg, ws, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        separate = e0.elapsed_time(e1) / args.steps
        plan.set_chained(True)
    if chain_err:
        raise SystemExit(f"bench: chained launch reported error {chain_err}")

    # second pass of the same length with per-launch HIP events: each
    # kernel over the whole set in its own launch
    plan.set_timing(1)
    plan.kernel_times()
    for _ in range(args.steps):
        plan.step(cfg, ws, stream)
    torch.cuda.synchronize()
    kt = plan.kernel_times()
    # and, for a chained plan, a third pass timed as it runs: events around
    # the momentum slot, the normalise slot and the chained launch
    as_run = None
    if chained:
        plan.set_timing(2)
        plan.kernel_times()
        plan.chain_times()
        for _ in range(args.steps):
            plan.step(cfg, ws, stream)
        torch.cuda.synchronize()
        kr = plan.kernel_times()
        c_ms, c_n = plan.chain_times()
        as_run = {"momentum": kr["momentum"], "normalize": kr["normalize"], "chain": (c_ms, c_n)}
    plan.set_timing(0)

    # one rank's share of an 8-GPU data-parallel step: the matrices rank 0
    # owns (ownership by algorithmic flops), through the same library; the
    # reduce-scatter and all-gather around it need more GPUs than this run has
    from workloads import matrix_flops, owner_split
    world_d = 8
    share = owner_split(wl.shapes, world_d)[0]
    splan = mu.MuonPlan([grads[i] for i in share], [bufs[i] for i in share] if bufs else None,
                        [outs[i] for i in share])
    sws = torch.empty(splan.workspace_bytes, dtype=torch.uint8, device=dev)
    s_steps = max(10, args.steps // 2)
    for _ in range(3):
        splan.step(cfg, sws, stream)
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for _ in range(s_steps):
        splan.step(cfg, sws, stream)
    s1.record(stream)
    torch.cuda.synchronize()
    s_ms = s0.elapsed_time(s1) / s_steps
    s_falg = wl.steps * sum(matrix_flops(*wl.shapes[i]) for i in share)
    s_bytes = sum(grads[i].numel() * grads[i].element_size() for i in share)
    splan.destroy()
    del sws

    # the next row beside the path: the same step with the weight application
    # fused into the last update (W read and written instead of out written)
    gen = torch.Generator(device="cpu").manual_seed(1234)
    weights = [(0.02 * torch.randn(g.shape, generator=gen)).to(g.dtype).to(dev) for g in grads]
    plan.set_weights(weights)
    n_apply = max(5, args.steps // 5)

    def block(fn):  # mean ms of n_apply calls, events on the step's stream
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for _ in range(n_apply):
            fn()
        b1.record(stream)
        torch.cuda.synchronize()
        return b0.elapsed_time(b1) / n_apply

    def plain():
        plan.step(cfg, ws, stream)

    def fused():
        plan.step_apply(cfg, 1e-3, 0.1, ws, stream)

    fused()
    plain()
    torch.cuda.synchronize()
    pairs = [(block(plain), block(fused)) for _ in range(3)]  # alternating blocks
    ms_plain_b = float(np.median([p for p, _ in pairs]))
    ms_apply = float(np.median([f for _, f in pairs]))
    del weights

    # the other half of the optimizer step: Adam over GPT-2 124M's parameters
    # off the Muon path (bf16 parameters, fp32 moments), one launch per step
    from workloads import gpt2_124m_adam_multipliers, gpt2_124m_adam_shapes, make_adam_state
    a_shapes = gpt2_124m_adam_shapes()
    a_lrm, a_wdm = gpt2_124m_adam_multipliers(a_shapes)
    ap, ag, am, av = make_adam_state(a_shapes, torch.bfloat16, 7, dev)
    aplan = mu.AdamPlan(ap, ag, am, av, a_lrm, a_wdm)
    a_steps = max(10, args.steps // 2)
    for t in range(1, 4):
        aplan.step(1e-3, 0.9, 0.99, 1e-8, 0.1, t, stream)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for t in range(4, 4 + a_steps):
        aplan.step(1e-3, 0.9, 0.99, 1e-8, 0.1, t, stream)
    c1.record(stream)
    torch.cuda.synchronize()
    a_us = c0.elapsed_time(c1) / a_steps * 1e3
    a_elems = sum(p.numel() for p in ap)
    a_bytes = a_elems * (2 + 2 + 4 + 4 + 2 + 4 + 4)  # read p, g, m, v; write p, m, v
    aplan.destroy()
    del ap, ag, am, av

    falg = wl.falg_flops()
    value = falg / (ms * 1e-3) / 1e12
    work = kernel_work(wl.shapes, wl.steps, wl.dtype)
    per_kernel = {}
    for name, (tot_ms, n) in kt.items():
        if n == 0:
            continue
        step_s = tot_ms / args.steps * 1e-3
        flops, nbytes = work[name]
        ent = {"launches_per_step": n / args.steps, "us_per_step": step_s * 1e6,
               "GB/s": nbytes / step_s / 1e9 if nbytes else None}
        if flops:
            ent["TFLOP/s"] = flops / step_s / 1e12
        per_kernel[name] = ent
    # the dominant kernel of the step as it runs: the chained launch (every
    # Gram, poly and update tile) for a chained plan, else the kernel with
    # the largest share in the per-kernel pass
    times = as_run if as_run is not None else kt
    dom = max(times, key=lambda k: times[k][0])
    d_step = times[dom][0] / args.steps * 1e-3
    roof = roofline_of(*work[dom], d_step, wl.dtype)
    t_step = measured_traffic(wl.name, dom)
    n_launch = times[dom][1] / args.steps
    # HBM bytes per launch (the counter runs' per-step figure over the step's
    # launches of this kernel), null when taken on another kernel source
    roof["traffic"] = None if t_step is None else t_step / n_launch
    roof["traffic_per_step"] = t_step
    roof["kernel"] = dom
    roof["us_per_step"] = d_step * 1e6
    roof["launches_per_step"] = n_launch

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded spiked-Gaussian gradients, GPT-2 shapes)",
        "config": {"workload": wl.name, "matrices": wl.n_matrices,
                   "shapes": "48x768x768 + 12x768x3072 + 12x3072x768"
                   if wl.name == "gpt2_124m_matrix_set" else str(sorted(set(wl.shapes))),
                   "ns_steps": wl.steps, "coeffs": list(wl.coeffs), "momentum": wl.momentum,
                   "nesterov": wl.nesterov, "falg_gflop_per_step": falg / 1e9,
                   "schedule": "chained" if chained else "separate launches"},
        "pct_bf16_dense_peak": 100.0 * value / PEAK["bf16"],
        "matrices_per_s": wl.n_matrices / (ms * 1e-3),
        "step_ms": {"n": int(step_ms.size), "mean": float(step_ms.mean()),
                    "sd": float(step_ms.std(ddof=1)) if step_ms.size > 1 else 0.0,
                    "min": float(step_ms.min())},
        "wall_s_timed": wall,
        "hip_graph": hip_graph,
        "separate_launches_ms_per_step": separate,
        "kernels": per_kernel,
        "step_as_run_us": None if as_run is None else
        {k: v[0] / args.steps * 1e3 for k, v in as_run.items()},
        "roofline": roof,
        "next": {"rank_share": {
            "world": world_d, "rank": 0, "matrices": len(share),
            "shapes": sorted({tuple(wl.shapes[i]) for i in share}),
            "ms_per_step": s_ms, "steps": s_steps, "TFLOP/s": s_falg / (s_ms * 1e-3) / 1e12,
            "grad_bytes_owned": s_bytes,
            "note": "muon_step on one rank's matrices of an 8-way sharded step; the "
                    "reduce-scatter / all-gather around it are not run (one GPU)"},
            "weight_apply": {
            "ms_per_step": ms_apply, "steps": 3 * n_apply,
            "plain_ms_per_step_same_blocks": ms_plain_b,
            "extra_us_vs_plain_step": (ms_apply - ms_plain_b) * 1e3,
            "note": "muon_plan_step_apply: W <- W(1 - lr wd) - lr X fused into the last update"},
            "adam": {
                "workload": "gpt2_124m_non_matrix_params", "tensors": len(a_shapes),
                "elements": a_elems, "us_per_step": a_us, "steps": a_steps,
                "roofline": {"bound": "hbm", "achieved": a_bytes / (a_us * 1e-6) / 1e9,
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": a_bytes / (a_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                             "bytes_per_step": a_bytes}}},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    plan.destroy()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
