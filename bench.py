"""Benchmark of the MXFP4 MoE expert layer on one MI355X.

A step is one layer call (router, top-k, permutation, MXFP4 gate/up + SwiGLU,
MXFP4 down, combine) over one synthetic batch, through the C ABI's single
persistent launch.  Default workload: the speculative-verify block (T=8
tokens, d=7168, ffn=2048, 256 experts, top-8).  Inputs are resident in HBM
before timing; the expert weights are rotated over `--replicas` distinct
copies (distinct layers) so that consecutive steps never re-read bytes that
could still sit in the 256 MB Infinity Cache.

Prints ONE JSON line.  `value` is the achieved algorithmic HBM bandwidth
(bytes the layer must move / time per layer): every active expert's packed
codes and scales once, the router weights, x and the fp32 output.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/layer + achieved HBM GB/s (% of peak), MXFP4 MoE, 8-token verify block"
HBM_PEAK_GBS = 8000.0
MXFP4_PEAK_TFLOPS = 10100.0
KERNEL_SOURCES = ["mxfp4_moe_expert_router_amd/csrc/moe_layer.hip", "mxfp4_moe_expert_router_amd/csrc/moe_device.h"]


def kernel_hash() -> str:
    m = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            m.update(f.read())
    return m.hexdigest()[:16]


def git_sha():
    """The checked-out commit, or None where the tree carries no git metadata
    (a copy of the sources; the source hashes of the line still identify the
    kernel, the input generator and this script)."""
    if not os.path.isdir(os.path.join(ROOT, ".git")):
        return None
    import subprocess
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
    except (OSError, subprocess.SubprocessError):
        return None
    return r.stdout.strip() or None if r.returncode == 0 else None


def source_hash(rels) -> str:
    m = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            m.update(f.read())
    return m.hexdigest()[:16]


GENERATOR_SOURCES = ["synth/gen.c", "synth/synth.py", "tests/golden/seeds.json"]


def host_info() -> dict:
    """CPU model string and the cores this process may use (the GPU machine's host)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "cpu_count": os.cpu_count(), "usable_cores": usable}


def precondition(step, seconds: float, sync) -> dict:
    """Untimed layer calls for at least `seconds` of wall time before the
    warmup steps, so that the timed steps start in the GPU's steady clock and
    power state (a few calls leave the clocks ramping: with 5 warmup calls the
    first ~20 verify calls ran ~15% slower than the rest)."""
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(64):
            step(n)
            n += 1
        sync()
        if time.perf_counter() - t0 >= seconds:
            break
    return {"what": "untimed layer calls on the same inputs and weight replicas, before the warmup steps",
            "seconds": round(time.perf_counter() - t0, 3), "calls": n}


def pct(a, q) -> float:
    import numpy as np
    return float(np.percentile(a, q))


def traffic_record(workload: str):
    """HBM traffic per launch measured with rocprofv3 counters (profiles/), if
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_hash") != kernel_hash():
        return None
    return rec


def stream_read_ref(dev, stream, gib: int = 4, reps: int = 10) -> dict:
    """Plain streaming reads on the same GPU, outside the timed region: two of
    torch's reductions over a gib-GiB buffer (each reads every byte once; of
    the torch reductions tried on MI355X these were the fastest, ~6 TB/s,
    where a plain fp32 sum reached ~4), each the mean of reps calls timed with
    HIP events; the faster one is the reference.  What a read-only kernel
    reaches on this machine, next to the 8 TB/s peak."""
    import torch

    buf = torch.ones(gib << 28, dtype=torch.float32, device=dev)
    nbytes = buf.numel() * 4
    best = None
    for how, f in (("torch int64 sum", lambda: buf.view(torch.int64).sum()),
                   ("torch fp32 column sums [8192, n]", lambda: buf.view(8192, -1).sum(dim=0))):
        for _ in range(3):
            f()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            f()
        b.record(stream)
        torch.cuda.synchronize()
        gbs = nbytes / (a.elapsed_time(b) * 1e-3 / reps) / 1e9
        if best is None or gbs > best[0]:
            best = (gbs, how)
    del buf
    torch.cuda.empty_cache()
    return {"GBs": round(best[0], 1), "how": f"{best[1]} over a {gib} GiB buffer, mean of {reps} (the faster of two)"}


# Trace stamps of the persistent launch (MOE_OPT_TRACE): slot -> end of phase.
TRACE_PHASES = [("router", 1), ("topk_published", 7), ("topk_read", 2), ("permutation_and_split", 3),
                ("gate_up", 4), ("first_h", 8), ("down", 5), ("combine", 6)]


def trace_phases(moe, torch, np, dims, cfg, xt, wrt, reps_p, reps_s, out, ws, calls):
    """Untimed calls with the trace option; per phase the median over calls of
    the median and the maximum over workgroups of the phase's end, in us from
    the call's first workgroup start (wall clock, 100 MHz)."""
    G = moe.persistent_grid(dims, cfg.k)
    opts = moe.Options(moe.MOE_OPT_TRACE, 0, 0)
    rows, plain = [], []
    for j in range(calls):
        moe.forward(xt, wrt, reps_p[j % len(reps_p)], reps_s[j % len(reps_s)], cfg.k, out=out, workspace=ws,
                    dims=dims, options=opts)
        torch.cuda.synchronize()
        rows.append(moe.intermediates(ws, dims, cfg.k)["trace"][:G].cpu().numpy().astype(np.int64))
    if moe.status(ws) != moe.MOE_OK:
        raise RuntimeError("device watchdog fired during the traced calls")
    tr = np.stack(rows)  # [calls, G, slots]
    rel = (tr - tr[:, :, 0].min(axis=1)[:, None, None]) / 100.0
    res = {"calls": calls, "grid": G, "unit": "us from the first workgroup's start",
           "stat": "median over calls of (median over workgroups, max over workgroups)"}
    for name, slot in TRACE_PHASES:
        v = rel[:, :, slot]
        if (v < 0).any() or (v > 1e6).any():  # a stamp this variant does not write
            res[name] = None
            continue
        res[name] = [round(float(np.median(np.median(v, axis=1))), 1), round(float(np.median(v.max(axis=1))), 1)]
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first: the GPU clocks take some tens of ms of load to ramp up")
    ap.add_argument("--workload", default="verify",
                    choices=["tiny", "decode", "verify", "batched_verify", "dense",
                             "sweep_T4", "sweep_T16", "sweep_T22", "sweep_T32", "verify_shared", "quantize",
                             "stack_verify"])
    ap.add_argument("--layers", type=int, default=8, help="layers of the stack_verify workload")
    ap.add_argument("--precondition-s", type=float, default=1.5,
                    help="seconds of untimed layer calls before the warmup steps (steady clocks)")
    ap.add_argument("--replicas", type=int, default=4, help="distinct copies of the expert weights")
    ap.add_argument("--staged", action="store_true", help="time the one-launch-per-step path instead")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--phases", type=int, default=0, metavar="CALLS",
                    help="after the timed steps, this many untimed calls with the trace option: per-phase "
                         "wall-clock stamps of every workgroup, reported as \"phases\" in the line")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 3}))
        return

    if args.workload == "quantize":
        if args.gpus != 1:
            print(json.dumps({"error": "one GPU only", "n_gpus": args.gpus}))
            sys.exit(2)
        bench_quantize(args)
        return

    if args.workload == "stack_verify":
        if args.gpus != 1:
            print(json.dumps({"error": "one GPU only", "n_gpus": args.gpus}))
            sys.exit(2)
        bench_stack(args)
        return

    if args.gpus != 1:
        print(json.dumps({"error": "this layer runs on one GPU; multi-GPU sharding (expert or tensor parallel) "
                                   "is described in the design notes but not built", "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import mxfp4_moe_expert_router_amd as moe
    from synth import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.get_config(args.workload)
    t_gen = time.time()
    x, wr = synth.routing_inputs(cfg)
    p, s = synth.expert_weights(cfg)
    gen_s = time.time() - t_gen
    print(f"[bench] inputs generated in {gen_s:.1f} s (workload {args.workload})", file=sys.stderr, flush=True)

    xt = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    wrt = torch.from_numpy(wr).to(dev)
    pt0 = torch.from_numpy(p).to(dev)
    st0 = torch.from_numpy(s).to(dev)
    reps_p, reps_s = [pt0], [st0]
    for _ in range(max(1, args.replicas) - 1):
        reps_p.append(pt0.clone())
        reps_s.append(st0.clone())
    R = len(reps_p)
    dims = moe.LayerDims(cfg.T, cfg.d, cfg.F, cfg.E)
    ws = moe.alloc_workspace(dims, cfg.k, dev)
    out = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    wsb = ws.numel()

    def step(i):
        st = moe.forward_raw(dims, xt.data_ptr(), wrt.data_ptr(), reps_p[i % R].data_ptr(),
                             reps_s[i % R].data_ptr(), cfg.k, out.data_ptr(), ws.data_ptr(), wsb, sh,
                             staged=args.staged)
        if st != 0:
            raise moe.MoeError(st, "forward")

    pre = precondition(step, args.precondition_s, torch.cuda.synchronize)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if moe.status(ws) != moe.MOE_OK:
        raise RuntimeError("device watchdog fired during warmup")

    # timed region: K steps, per-launch HIP events on the launch stream
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step(args.warmup + i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if moe.status(ws) != moe.MOE_OK:
        raise RuntimeError("device watchdog fired during the timed steps")
    launch_ms = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])

    phases = None
    if args.phases > 0 and not args.staged:
        phases = trace_phases(moe, torch, np, dims, cfg, xt, wrt, reps_p, reps_s, out, ws, args.phases)

    ref = stream_read_ref(dev, stream)

    it = moe.intermediates(ws, dims, cfg.k)
    n_active = int(it["n_active"].item())
    alg_bytes = synth.algorithmic_bytes(cfg, n_active)
    flops = synth.layer_flops(cfg)
    ms_per_step = elapsed * 1e3 / args.steps
    us_layer = ms_per_step * 1e3
    gbs = alg_bytes / (ms_per_step * 1e-3) / 1e9
    kern_ms = float(np.median(launch_ms))
    kern_gbs = alg_bytes / (kern_ms * 1e-3) / 1e9

    traffic = None
    trec = traffic_record(args.workload + ("_staged" if args.staged else ""))
    if trec is not None:
        traffic = trec.get("hbm_bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "dtype_detail": "MXFP4 (E2M1 + E8M0) weights, bf16 activations, bf16x2 dot / fp32 FMA, fp32 accumulation",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: T={cfg.T} d={cfg.d} ffn={cfg.F} E={cfg.E} top-{cfg.k}"
                        + (f" Zipf(s={cfg.zipf_s})" if cfg.zipf_s else ""),
            "T": cfg.T, "d": cfg.d, "ffn": cfg.F, "E": cfg.E, "topk": cfg.k,
            "route_seed": cfg.route_seed, "active_experts": n_active,
            "weight_replicas": R, "path": "staged (one launch per step)" if args.staged else "persistent single launch",
        },
        "us_per_layer": round(us_layer, 2),
        "tokens_per_s_per_layer": round(cfg.T / (ms_per_step * 1e-3), 1),
        "algorithmic_bytes": alg_bytes,
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(kern_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "k_layer (the persistent launch)" if not args.staged else "every step's launch (staged)",
            "kernel_us_median": round(kern_ms * 1e3, 2),
            "kernel_us_p10": round(pct(launch_ms, 10) * 1e3, 2),
            "kernel_us_p90": round(pct(launch_ms, 90) * 1e3, 2),
            "kernel_us_mean": round(float(launch_ms.mean()) * 1e3, 2),
            "achieved_from": "algorithmic bytes / median launch duration (HIP events on the launch stream)",
            "mfma_frac_of_mxfp4_peak_if_all_flops_on_mfma": round(flops / (kern_ms * 1e-3) / 1e12
                                                                   / MXFP4_PEAK_TFLOPS, 5),
        },
        "kernel_hash": kernel_hash(),
        "generator_hash": source_hash(GENERATOR_SOURCES),
        "bench_hash": source_hash(["bench.py"]),
        "git_sha": git_sha(),
        "preconditioning": pre,
        "host": host_info(),
        "stream_read_ref": dict(ref, layer_kernel_frac=round(kern_gbs / ref["GBs"], 4)),
    }
    if phases is not None:
        result["phases"] = phases

    if not args.no_cpu_baseline:
        from oracle import oracle
        nth = args.cpu_threads or min(16, os.cpu_count() or 1)
        mask = None
        sample = f"the whole {args.workload} layer (all {cfg.T} tokens)"
        if cfg.T > 8:  # bound the CPU work: a sample of tokens, scaled per token
            mask = np.zeros(cfg.T, dtype=np.uint8)
            mask[:: max(1, cfg.T // 8)] = 1
            sample = f"{int(mask.sum())} of {cfg.T} tokens of the {args.workload} layer (all routing)"
        t1 = time.perf_counter()
        oracle.forward(x, wr, p, s, cfg.k, cfg.F, token_mask=mask, nthreads=nth)
        cpu_s = time.perf_counter() - t1
        frac = 1.0 if mask is None else float(mask.sum()) / cfg.T
        cpu_layer_s = cpu_s / frac
        result["cpu_baseline"] = {
            "value": round(alg_bytes / cpu_layer_s / 1e9, 4),
            "unit": "GB/s",
            "cores": nth,
            "kind": "oracle",
            "sample": sample + f"; fp64 C oracle, {cpu_s:.2f} s wall, {nth} OpenMP threads",
            "us_per_layer": round(cpu_layer_s * 1e6, 1),
            "cpu_model": result["host"]["cpu_model"],
        }
        if cfg.T <= 8:
            # one thread, on one token of the block (all routing, that token's
            # expert pairs), scaled per token
            m1 = np.zeros(cfg.T, dtype=np.uint8)
            m1[0] = 1
            t1 = time.perf_counter()
            oracle.forward(x, wr, p, s, cfg.k, cfg.F, token_mask=m1, nthreads=1)
            s1 = (time.perf_counter() - t1) * cfg.T
            result["cpu_baseline"]["single_thread"] = {
                "value": round(alg_bytes / s1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                "us_per_layer": round(s1 * 1e6, 1),
                "sample": f"token 0 of {cfg.T} (all routing, its {cfg.k} expert pairs), one thread, "
                          f"{s1 / cfg.T:.2f} s wall, scaled by {cfg.T} tokens"}
    print(json.dumps(result), flush=True)


def bench_stack(args):
    """A stack of L verify-block layers on one residual stream
    (moe_mxfp4_forward_layers), timed three ways: one launch per operator (per
    layer the input normalisation, then the layer; the library's default and
    `value`), the whole stack in one resident launch, and the per-operator
    launches captured once in a HIP graph and replayed.  Layer l has its own router weights and
    its own copy of the experts (layer 0's, relabelled by 37 l), so no layer
    re-reads another's bytes.  Algorithmic bytes: the sum over layers of the
    lone layer's (each layer's own active experts, found by running the
    prefixes of the stack once)."""
    import numpy as np
    import torch

    import mxfp4_moe_expert_router_amd as moe
    from synth import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = args.layers
    base = synth.get_config("verify")
    t_gen = time.time()
    x, _ = synth.routing_inputs(base)
    p0, s0 = synth.expert_weights(base)
    wr = np.stack([synth.routing_inputs(synth.chain_layer_config(base, l))[1] for l in range(L)])
    print(f"[bench] inputs generated in {time.time() - t_gen:.1f} s (stack of {L})", file=sys.stderr, flush=True)
    xt = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    wrt = torch.from_numpy(wr).to(dev)
    pt0 = torch.from_numpy(p0).to(dev)
    st0 = torch.from_numpy(s0).to(dev)
    pt = torch.stack([torch.roll(pt0, -37 * l, dims=0) for l in range(L)])
    st = torch.stack([torch.roll(st0, -37 * l, dims=0) for l in range(L)])
    del pt0, st0
    dims = moe.LayerDims(base.T, base.d, base.F, base.E)
    ws = moe.alloc_workspace(dims, base.k, dev)
    out = torch.empty((base.T, base.d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    wsb = ws.numel()
    one = moe.layers_one_launch(dims, base.k)

    # every layer's active experts: the last layer of each prefix of the stack
    n_active = []
    for l in range(L):
        moe.forward_layers(xt, wrt[: l + 1], pt[: l + 1], st[: l + 1], base.k, out=out, workspace=ws,
                           flags=moe.MOE_LAYERS_PER_LAUNCH, dims=dims)
        n_active.append(int(moe.intermediates(ws, dims, base.k)["n_active"].item()))
    alg_bytes = sum(synth.algorithmic_bytes(base, n) for n in n_active)

    def call(flags, s_handle):
        r = moe.forward_layers_raw(dims, L, xt.data_ptr(), wrt.data_ptr(), pt.data_ptr(), st.data_ptr(), base.k,
                                   out.data_ptr(), ws.data_ptr(), wsb, flags, s_handle)
        if r != 0:
            raise moe.MoeError(r, "forward_layers")

    def timed(run, warm):
        for _ in range(warm):
            run()
        torch.cuda.synchronize()
        if moe.status(ws) != moe.MOE_OK:
            raise RuntimeError("device watchdog fired")
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        t0 = time.perf_counter()
        for a, b in ev:
            a.record(stream)
            run()
            b.record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / args.steps
        if moe.status(ws) != moe.MOE_OK:
            raise RuntimeError("device watchdog fired")
        ms = np.array([a.elapsed_time(b) for a, b in ev])
        return wall, ms

    sh = stream.cuda_stream
    modes = {}
    warm = max(1, args.warmup // L)
    if one:
        modes["one_launch"] = timed(lambda: call(moe.MOE_LAYERS_ONE_LAUNCH, sh), warm)
        ref_out = out.clone()
    modes["launch_per_operator"] = timed(lambda: call(moe.MOE_LAYERS_PER_LAUNCH, sh), warm)
    same = bool(torch.equal(ref_out, out)) if one else None
    # the per-layer launches captured once, replayed
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream(dev)
    cs.wait_stream(stream)
    with torch.cuda.stream(cs):
        call(moe.MOE_LAYERS_PER_LAUNCH, cs.cuda_stream)  # warm the library's per-device set-up outside capture
    stream.wait_stream(cs)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cs):
        call(moe.MOE_LAYERS_PER_LAUNCH, cs.cuda_stream)
    torch.cuda.synchronize()
    modes["graph_replay"] = timed(lambda: g.replay(), warm)
    graph_same = bool(torch.equal(ref_out, out)) if one else None

    main_mode = "launch_per_operator"  # the library's default
    wall, ms = modes[main_mode]
    kern_s = float(ms.mean()) * 1e-3
    result = {
        "metric": METRIC,
        "value": round(alg_bytes / wall / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warm,
        "ms_per_step": round(wall * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "dtype_detail": "MXFP4 (E2M1 + E8M0) weights, bf16 activations, bf16x2 dot / fp32 FMA, fp32 accumulation",
        "data": "synthetic",
        "config": {
            "workload": f"stack_verify: {L} layers of T={base.T} d={base.d} ffn={base.F} E={base.E} top-{base.k} "
                        f"on one residual stream",
            "T": base.T, "d": base.d, "ffn": base.F, "E": base.E, "topk": base.k, "layers": L,
            "active_experts_per_layer": n_active, "path": main_mode.replace("_", " "),
        },
        "us_per_layer": round(wall * 1e6 / L, 2),
        "algorithmic_bytes": alg_bytes,
        "modes_us_per_stack": {k: {"wall": round(v[0] * 1e6, 2), "events_mean": round(float(v[1].mean()) * 1e3, 2),
                                   "events_p10": round(float(np.percentile(v[1], 10)) * 1e3, 2),
                                   "events_p90": round(float(np.percentile(v[1], 90)) * 1e3, 2)}
                               for k, v in modes.items()},
        "one_launch_equals_per_operator": same,
        "graph_equals_one_launch": graph_same,
        "roofline": {
            "bound": "hbm", "achieved": round(alg_bytes / kern_s / 1e9, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(alg_bytes / kern_s / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "k_norm + k_layer per layer (events around the stack call)",
            "kernel_us_mean": round(kern_s * 1e6, 2),
        },
        "kernel_hash": kernel_hash(),
        "git_sha": git_sha(),
    }
    if not args.no_cpu_baseline:
        from oracle import oracle
        nth = args.cpu_threads or min(16, os.cpu_count() or 1)
        t1 = time.perf_counter()
        oracle.forward(x, wr[0], p0, s0, base.k, base.F, nthreads=nth)
        cpu_s = time.perf_counter() - t1
        alg0 = synth.algorithmic_bytes(base, n_active[0])
        result["cpu_baseline"] = {"value": round(alg0 / cpu_s / 1e9, 4), "unit": "GB/s", "cores": nth,
                                  "kind": "oracle",
                                  "sample": f"layer 0 of the stack (all {base.T} tokens); fp64 C oracle, "
                                            f"{cpu_s:.2f} s wall, {nth} OpenMP threads"}
    print(json.dumps(result), flush=True)


def bench_quantize(args):
    """MXFP4 quantize/pack (moe_mxfp4_quantize) of 16 experts' worth of fp32
    weights (16 x 3 x 2048 rows of 7168 values, N(0, 0.02)), device resident.
    Algorithmic bytes: 4 per value read, 0.5 + 1/32 per value written."""
    import numpy as np
    import torch

    import mxfp4_moe_expert_router_amd as moe

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rows, K = 16 * 3 * 2048, 7168
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    w = torch.randn((rows, K), generator=gen, device=dev, dtype=torch.float32).mul_(0.02)
    packed = torch.empty((rows, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        moe.quantize(w, packed, scales)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        moe.quantize(w, packed, scales)
        ends[i].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    n = rows * K
    alg = n * 4 + n // 2 + n // 32
    kern_s = float(ms.mean()) * 1e-3
    step_s = elapsed / args.steps
    # the same weights as bf16 input (2 bytes per value read), kernel time only
    wb = w.to(torch.bfloat16)
    for _ in range(args.warmup):
        moe.quantize(wb, packed, scales)
    torch.cuda.synchronize()
    for i in range(args.steps):
        starts[i].record(stream)
        moe.quantize(wb, packed, scales)
        ends[i].record(stream)
    torch.cuda.synchronize()
    kern_b = float(np.mean([a.elapsed_time(b) for a, b in zip(starts, ends)])) * 1e-3
    alg_b = n * 2 + n // 2 + n // 32
    del wb
    result = {
        "metric": "achieved HBM GB/s (% of peak), MXFP4 quantize/pack of fp32 weights on the GPU",
        "value": round(alg / step_s / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "dtype_detail": "fp32 in, E2M1 codes + E8M0 scales out; every code exact (the rounding rule's own result)",
        "data": "synthetic",
        "config": {"workload": f"quantize: {rows} x {K} fp32 (16 experts of d=7168, ffn=2048)", "rows": rows, "K": K},
        "algorithmic_bytes": alg,
        "roofline": {"bound": "hbm", "achieved": round(alg / kern_s / 1e9, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(alg / kern_s / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "k_quantize<false>", "kernel_us_mean": round(kern_s * 1e6, 2)},
        "bf16_input": {"kernel": "k_quantize<true>", "kernel_us_mean": round(kern_b * 1e6, 2),
                       "algorithmic_bytes": alg_b, "achieved": round(alg_b / kern_b / 1e9, 2),
                       "frac": round(alg_b / kern_b / 1e9 / HBM_PEAK_GBS, 4)},
    }
    if not args.no_cpu_baseline:
        from oracle import oracle
        sr = 256  # a sample of rows, scaled per value
        ws = w[:sr].double().cpu().numpy()
        t1 = time.perf_counter()
        oracle.quantize(ws)
        cpu_s = (time.perf_counter() - t1) * rows / sr
        result["cpu_baseline"] = {"value": round(alg / cpu_s / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                                  "sample": f"{sr} of {rows} rows, single-threaded C oracle, scaled per value"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
