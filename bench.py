#!/usr/bin/env python3
"""Throughput of the MoE-layer hot path on one MI355X.

One step is one call of moe_layer_forward (router, top-k and gates, slots,
bucket scatter, grouped SwiGLU GEMMs, combine) over one batch of tokens, with
inputs and weights already resident in HBM. Default workload: the
Mixtral-shaped prefill layer (T=4096 tokens, d=4096, E=8 experts, top-2,
d_ff=14336, cf=1.25, bf16), synthetic seeded inputs.

Prints one JSON line: routed tokens/s per layer (whole job), per-stage GPU
times from HIP events recorded by the library around each stage, the
roofline of the dominant kernel, and the CPU oracle timed on a bounded sample
of the same workload.

With --replicas EXTRA a step is one call of moe_layer_forward_replicated,
with EXTRA replicas dealt to the most loaded experts of the same batch.

With --backward a step is one call of moe_layer_backward instead (the
gradients of x, the router and the expert weights for a seeded dout), and the
line reports backward tokens/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
METRIC = "routed tokens/s per MoE layer; grouped-GEMM % MFMA peak; permute % HBM BW"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_gate_up_mixtral_prefill_traffic.txt")
GEMM_SOURCE = os.path.join(ROOT, "routing_dispatch_expert_amd", "csrc", "grouped_gemm.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_prefill")
    ap.add_argument("--cpu-sample", type=int, default=4096, help="tokens whose output the oracle computes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-stage event loop")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="in the per-stage loop, read this many MiB before each step so that L2 and the "
                         "Infinity Cache hold nothing of the layer's data (0: no flush)")
    ap.add_argument("--backward", action="store_true", help="time moe_layer_backward instead of the forward")
    ap.add_argument("--replicas", type=int, default=-1, metavar="EXTRA",
                    help="time moe_layer_forward_replicated with EXTRA replicas dealt greedily to the most loaded "
                         "experts (counts from one plain forward of the same batch)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first copy a buffer of this many MiB on the device (a reference kernel of known "
                         "traffic for hardware counters)")
    return ap.parse_args()


def stage_work(wl, n_kept: int, touched: int, buckets: int):
    """Algorithmic HBM bytes (and flops) of each stage for this run: kept rows
    only, touched buckets' weights only (a replicated expert's weights once
    per instance, as each instance would hold its own copy), every operand
    moved once. buckets = E, or the instance count R when replicated."""
    T, d, f, E, k = wl.T, wl.d, wl.d_ff, wl.E, wl.k
    b = wl.elem_bytes
    nt = -(-T // 64)
    return {
        "router": dict(bytes=T * d * b + E * d * b + T * E * 4, flops=2 * T * d * E, bound="hbm"),
        "route": dict(bytes=T * E * 4 + T * k * 8, flops=0, bound="hbm"),
        "slots": dict(bytes=3 * T * k * 4 + 4 * nt * buckets * 4, flops=0, bound="hbm"),
        "scatter": dict(bytes=(T + n_kept) * d * b + T * k * 8, flops=0, bound="hbm"),
        "gate_up": gemm_work(touched * 2 * f * d * b + n_kept * (d + f) * b, 4 * n_kept * d * f, wl.dtype),
        "down": gemm_work(touched * f * d * b + n_kept * (f + d) * b, 2 * n_kept * d * f, wl.dtype),
        "combine": dict(bytes=(n_kept + 2 * T) * d * b + T * k * 12, flops=0, bound="hbm"),
    }


def gemm_work(nbytes: int, flops: int, dtype: str):
    """A GEMM stage is bound by the matrix cores when its arithmetic intensity
    is above the ridge point (peak flop/s over peak HBM bytes/s), else by HBM."""
    ridge = PEAK_TFLOPS[dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    return dict(bytes=nbytes, flops=flops, bound="mfma" if flops >= ridge * nbytes else "hbm")


def read_traffic(gemm_src_sha: str):
    """HBM bytes per launch of the gate/up GEMM from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    txt = open(TRAFFIC_FILE).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not (m_sha and m_b) or m_sha.group(1) != gemm_src_sha:
        return None
    return float(m_b.group(1))


def cpu_baseline(wl, host_w, sample: int, replicas=None):
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    tokens = np.arange(min(sample, wl.T))
    times = []
    for _ in range(3):  # median of three runs
        t0 = time.perf_counter()
        oracle.layer_forward(wl.x, wl.wr, lambda e: (host_w[0][e], host_w[1][e], host_w[2][e]), wl.T, wl.d,
                             wl.d_ff, wl.E, wl.k, wl.cf, wl.dtype, P=wl.P, bias=wl.bias_vec, tokens=tokens,
                             max_ranks=wl.max_ranks, replicas=replicas)
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[1]
    return {"value": round(tokens.size / dt, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "host": host_cpu(),
            "sample": f"layer outputs of the first {tokens.size} of {wl.T} tokens (routing and slots of all "
                      f"{wl.T}), fp64 numpy, median of 3 runs: {dt:.1f} s each ({sum(times):.1f} s total)"}


def run_backward(args, wl, moe, torch, np, dev, to_dev, host_w):
    """One step = moe_layer_backward over the workload, inputs resident in HBM."""
    x, wr = to_dev(wl.x), to_dev(wl.wr)
    wg, wu, wd = (to_dev(a) for a in host_w)
    dout = to_dev(wl.grad_out(1))
    bias = None if wl.bias_vec is None else torch.from_numpy(wl.bias_vec).to(dev)
    T, d, d_ff, E, k, cf, P = wl.T, wl.d, wl.d_ff, wl.E, wl.k, wl.cf, wl.P
    outs = {"dx": torch.empty_like(x), "dW_router": torch.empty_like(wr), "dW_gate": torch.empty_like(wg),
            "dW_up": torch.empty_like(wu), "dW_down": torch.empty_like(wd),
            "d_bias": torch.empty(E, dtype=torch.float32, device=dev)}
    ws_bytes = moe.moe_backward_workspace_size(T, d, d_ff, E, k, cf, P, wl.dtype)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        moe.moe_layer_backward(x, wr, bias, wg, wu, wd, dout, T, d, d_ff, E, k, cf, P, wl.max_ranks, wl.dtype,
                               outs["dx"], outs["dW_router"], outs["d_bias"], outs["dW_gate"], outs["dW_up"],
                               outs["dW_down"], ws, ws_bytes, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1) / args.steps
    print(f"[bench] backward: timed {args.steps} steps: {wall * 1e3 / args.steps:.3f} ms/step wall, "
          f"{gpu_ms:.3f} ms/step GPU", file=sys.stderr, flush=True)
    import oracle
    r = oracle.layer_forward(wl.x, wl.wr, lambda e: (host_w[0][e], host_w[1][e], host_w[2][e]), T, d, d_ff, E, k,
                             cf, wl.dtype, P=P, bias=wl.bias_vec, tokens=np.arange(0), max_ranks=wl.max_ranks)
    n_kept = int(r["kept"].sum())
    algo = 12 * n_kept * d * d_ff  # dh, dX (two), dWd, dWg, dWu: 2 N d d_ff flop each
    done = algo + 4 * n_kept * d * d_ff  # plus the recomputed g and u
    tf = algo / gpu_ms / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        S = min(args.cpu_sample, T, 1024)  # the fp64 backward costs about 3x the forward per token
        sub = moe_inputs_sample(wl, S)
        print(f"[bench] timing the CPU oracle backward on {S} tokens", file=sys.stderr, flush=True)
        times = []
        for _ in range(3):
            t1 = time.perf_counter()
            oracle.layer_backward(sub["x"], wl.wr, lambda e: (host_w[0][e], host_w[1][e], host_w[2][e]), sub["dout"],
                                  S, d, d_ff, E, k, cf, wl.dtype, P=P, bias=wl.bias_vec, max_ranks=wl.max_ranks)
            times.append(time.perf_counter() - t1)
        dt = sorted(times)[1]
        cpu = {"value": round(S / dt, 3), "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
               "host": host_cpu(),
               "sample": f"backward of the first {S} of {T} tokens as a layer of their own (capacity for {S} "
                         f"tokens), fp64 numpy, median of 3 runs: {dt:.1f} s each"}
    line = {
        "metric": "backward tokens/s per MoE layer (gradients of x, router and expert weights)",
        "value": round(T * args.steps / wall, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded Gaussian inputs, upstream gradient and random-init weights of the named shape)",
        "config": {"workload": wl.name, "T": T, "d": d, "E": E, "k": k, "d_ff": d_ff, "cf": cf, "P": P,
                   "max_ranks": wl.max_ranks, "N_kept": n_kept},
        "gpu_ms_per_step": round(gpu_ms, 4),
        "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_TFLOPS[wl.dtype], "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_TFLOPS[wl.dtype], 4), "traffic": None,
                     "kernel": "whole backward step (expert-gradient flops over step time)",
                     "algo_flops_per_step": algo, "executed_gemm_flops_per_step": done},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def moe_inputs_sample(wl, S):
    """The first S tokens (and their upstream gradient) as a layer input."""
    return {"x": wl.x[:S], "dout": wl.grad_out(1)[:S]}


def host_cpu():
    """The host's CPU model and logical CPU count, for the oracle's timing."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "logical_cpus": os.cpu_count()}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1]))
    except Exception:  # pragma: no cover
        return 1


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the layer here has no multi-GPU path (asked for --gpus "
              f"{args.gpus})", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import moe_inputs
    import routing_dispatch_expert_amd as moe

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    moe.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = moe_inputs.workload(args.workload)
    print(f"[bench] workload {wl.name}: T={wl.T} d={wl.d} E={wl.E} k={wl.k} d_ff={wl.d_ff} cf={wl.cf} "
          f"P={wl.P} {wl.dtype}", file=sys.stderr, flush=True)

    def to_dev(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    host_w = wl.all_expert_weights()
    if args.backward:
        run_backward(args, wl, moe, torch, np, dev, to_dev, host_w)
        return
    x, wr = to_dev(wl.x), to_dev(wl.wr)
    wg, wu, wd = (to_dev(a) for a in host_w)
    bias = None if wl.bias_vec is None else torch.from_numpy(wl.bias_vec).to(dev)
    T, d, d_ff, E, k, cf, P = wl.T, wl.d, wl.d_ff, wl.E, wl.k, wl.cf, wl.P
    C = moe.moe_capacity(T, E, k, cf)
    i32 = dict(dtype=torch.int32, device=dev)
    outs = {"out": torch.empty_like(x), "topk_idx": torch.empty((T, k), **i32),
            "topk_w": torch.empty((T, k), dtype=torch.float32, device=dev), "slot": torch.empty((T, k), **i32),
            "routed_count": torch.empty(E, **i32), "kept_count": torch.empty(E, **i32),
            "send_count": torch.empty(P, **i32), "totals": torch.empty(4, dtype=torch.int64, device=dev)}
    ws_bytes = moe.moe_workspace_size(T, d, d_ff, E, k, cf, P, wl.dtype)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        moe.moe_layer_forward(x, wr, bias, wg, wu, wd, T, d, d_ff, E, k, cf, P, wl.max_ranks, wl.dtype, outs["out"],
                              outs, ws, ws_bytes, stream)

    reps, repl_cfg = None, {}
    if args.replicas >= 0:
        step()
        torch.cuda.synchronize()
        base_dropped = int(outs["totals"][0].item())
        reps = moe.moe_replica_plan(outs["routed_count"].cpu().numpy(), args.replicas)
        R = int(reps.sum())
        reps_dev = torch.from_numpy(reps).to(dev)
        outs["kept_count"] = torch.empty(R, **i32)
        outs["instance"] = torch.empty((T, k), **i32)
        ws_bytes = moe.moe_replicated_workspace_size(T, d, d_ff, E, k, cf, P, R, wl.dtype)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        repl_cfg = {"replicas_extra": args.replicas, "instances": R, "replicated_experts": int((reps > 1).sum()),
                    "max_replicas": int(reps.max()), "dropped_without_replicas": base_dropped}
        print(f"[bench] replicated layer: {R} instances, replicas {reps.tolist()}", file=sys.stderr, flush=True)

        def step():  # noqa: F811 (the replicated layer replaces the plain one)
            moe.moe_layer_forward_replicated(x, wr, bias, wg, wu, wd, T, d, d_ff, E, k, cf, P, wl.max_ranks, reps_dev,
                                             R, wl.dtype, outs["out"], outs, ws, ws_bytes, stream)

    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1) / args.steps
    print(f"[bench] timed {args.steps} steps: {wall * 1e3 / args.steps:.3f} ms/step wall, {gpu_ms:.3f} ms/step "
          f"GPU", file=sys.stderr, flush=True)

    kept = outs["kept_count"].cpu().numpy()
    n_kept, touched = int(kept.sum()), int((kept > 0).sum())
    totals = outs["totals"].cpu().numpy().tolist()
    work = stage_work(wl, n_kept, touched, int(kept.size))

    stages = {}
    if not args.no_profile:
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(moe.STAGES))]
        for e in evs:
            e.record(stream)           # creates the underlying hipEvent_t
        torch.cuda.synchronize()
        moe.moe_set_stage_events([e.cuda_event for e in evs])
        acc = np.zeros(len(moe.STAGES))
        layer_ms = []
        # a read, not a write: evicting dirty lines would add write-back traffic to the next step
        flush = torch.ones((args.flush_mib << 20) // 8, dtype=torch.int64, device=dev) if args.flush_mib else None
        try:
            for n in range(args.steps):
                if flush is not None:
                    flush.sum()
                step()
                torch.cuda.synchronize()
                acc += [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(len(moe.STAGES))]
                layer_ms.append(evs[0].elapsed_time(evs[-1]))
        finally:
            moe.moe_set_stage_events(None)
        del flush
        for i, name in enumerate(moe.STAGES):
            ms = acc[i] / args.steps
            w = work[name]
            s = {"ms": round(ms, 5), "algo_bytes": int(w["bytes"]),
                 "GB_per_s": round(w["bytes"] / ms / 1e6, 1) if ms > 0 else None,
                 "hbm_frac": round(w["bytes"] / ms / 1e6 / PEAK_HBM_GBS, 4) if ms > 0 else None}
            if w["flops"]:
                s["TFLOP_per_s"] = round(w["flops"] / ms / 1e9, 1) if ms > 0 else None
                s["mfma_frac"] = round(w["flops"] / ms / 1e9 / PEAK_TFLOPS[wl.dtype], 4) if ms > 0 else None
            stages[name] = s
            print(f"[bench] stage {name:8s} {ms:8.4f} ms  " + " ".join(f"{a}={b}" for a, b in s.items()
                                                                       if a != "ms"), file=sys.stderr, flush=True)

    roofline = None
    if stages:
        dom = max(stages, key=lambda n: stages[n]["ms"])
        w, s = work[dom], stages[dom]
        sha = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
        traffic = read_traffic(sha) if (dom == "gate_up" and wl.name == "mixtral_prefill") else None
        if w["bound"] == "mfma":
            roofline = {"bound": "mfma", "achieved": s["TFLOP_per_s"], "peak": PEAK_TFLOPS[wl.dtype],
                        "unit": "TFLOP/s", "frac": s["mfma_frac"], "traffic": traffic, "kernel": dom,
                        "algo_flops_per_launch": int(w["flops"]), "avg_launch_ms": s["ms"]}
        else:
            roofline = {"bound": "hbm", "achieved": s["GB_per_s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": s["hbm_frac"], "traffic": traffic, "kernel": dom,
                        "algo_bytes_per_launch": int(w["bytes"]), "avg_launch_ms": s["ms"]}

    layer_cold = None
    if stages:
        layer_cold = round(float(np.median(layer_ms)), 5)
        print(f"[bench] layer (first to last kernel, after a {args.flush_mib} MiB read): median {layer_cold} ms",
              file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle on {min(args.cpu_sample, T)} tokens", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, host_w, args.cpu_sample, reps)

    metric = METRIC if reps is None else METRIC + " (hot experts replicated)"
    line = {
        "metric": metric, "value": round(T * args.steps / wall, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded Gaussian inputs and random-init weights of the named shape)",
        "config": {"workload": wl.name, "T": T, "d": d, "E": E, "k": k, "d_ff": d_ff, "cf": cf, "P": P,
                   "max_ranks": wl.max_ranks, "C": C, "N_kept": n_kept, "touched_experts": touched,
                   "dropped": totals[0], **repl_cfg},
        "gpu_ms_per_step": round(gpu_ms, 4),
        "assignments_per_s": round(T * k * args.steps / wall, 1),
        "layer_ms_cold_median": layer_cold,
        "stage_timing": None if not stages else (
            f"HIP events around each stage, mean of {args.steps} steps, each after a {args.flush_mib} MiB read "
            "that leaves none of the layer's data in L2 or the Infinity Cache"),
        "grouped_gemm_mfma_frac": None if not stages else round(
            (work["gate_up"]["flops"] + work["down"]["flops"]) /
            ((stages["gate_up"]["ms"] + stages["down"]["ms"]) * 1e9) / PEAK_TFLOPS[wl.dtype], 4),
        "permute_hbm_frac": None if not stages else stages["scatter"]["hbm_frac"],
        "combine_hbm_frac": None if not stages else stages["combine"]["hbm_frac"],
        "stages": stages, "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
