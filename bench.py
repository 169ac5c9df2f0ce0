#!/usr/bin/env python3
"""Throughput of the MoE-layer hot path on one MI355X.

One step is one call of moe_layer_forward (router, top-k and gates, slots,
bucket scatter, grouped SwiGLU GEMMs, combine) over one batch of tokens, with
inputs and weights already resident in HBM. Default workload: the
DeepSeek-V3-shaped prefill layer (T=8192 tokens, d=7168, E=256 experts, top-8,
d_ff=2048, cf=1.25, bf16, buckets laid out as P=8 send buffers), synthetic
seeded inputs; --workload names another (mixtral_prefill, zipf_skew_drops,
deepseek_v3_decode, deepseek_v3_node_limited, tiny_f32).

Prints one JSON line: routed tokens/s per layer (whole job), per-stage GPU
times from HIP events recorded by the library around each stage, the
roofline of the dominant kernel, and the CPU oracle timed on a bounded sample
of the same workload.

With --graph the timed steps are replays of one layer call captured in a HIP
graph (the library allocates nothing and never waits on the host, so a call
can be captured as it is); the per-stage event steps stay eager.

With --replicas EXTRA a step is one call of moe_layer_forward_replicated,
with EXTRA replicas dealt to the most loaded experts of the same batch.

With --backward a step is one call of moe_layer_backward instead (the
gradients of x, the router and the expert weights for a seeded dout), and the
line reports backward tokens/s. With --saved as well, a step is one call of
moe_layer_backward_saved on the state of a forward that kept its
activations; the line also gives that forward's time and that of the two
together.

With --counters-summary no GPU work is done: the rocprofv3 counter CSVs of
the profiling passes (PROFILE_PASSES, each a run of this script under
rocprofv3 --pmc) are summarised per kernel, in the text format of the
profiles/*_counters.txt files that the roofline's `traffic` is read from.
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
DEFAULT_WORKLOAD = "deepseek_v3_prefill"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "routing_dispatch_expert_amd", "csrc")
# the sources a kernel's counters depend on (the summary is stale once they change)
STAGE_SOURCES = {"gate_up": ["grouped_gemm.hip", "common.h"], "down": ["grouped_gemm.hip", "common.h"],
                 "scatter": ["permute.hip", "common.h"], "combine": ["combine.hip", "common.h"]}
# tokens whose layer output the CPU oracle computes for the baseline (all when absent)
CPU_SAMPLE = {"deepseek_v3_prefill": 512, "deepseek_v3_node_limited": 512}
# rocprofv3 counter passes, one run each: name, counters (within one pass's
# hardware limits: FETCH_SIZE takes 3 TCC counters, WRITE_SIZE 2)
PROFILE_PASSES = [("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE"),
                  ("mfma", "MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_WAVE_CYCLES SQ_WAIT_INST_ANY "
                           "SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS GRBM_GUI_ACTIVE"),
                  ("l2", "TCC_HIT_sum TCC_MISS_sum")]
PROFILE_CMD = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 --pmc {counters} --output-format csv "
               "-d $OUT/{workload}/{name} -o run -- python $REPO/bench.py --workload {workload} --steps 2 --warmup 1 "
               "--no-cpu-baseline --no-profile --device-weights --copy-probe-mib 1024")
COPY_PROBE_KIB = 1024 * 1024


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="tokens whose output the oracle computes (default: all, or 512 on the DeepSeek-V3 "
                         "prefill shapes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-stage event loop")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="in the per-stage loop, read this many MiB before each step so that L2 and the "
                         "Infinity Cache hold nothing of the layer's data (0: no flush)")
    ap.add_argument("--backward", action="store_true", help="time moe_layer_backward instead of the forward")
    ap.add_argument("--saved", action="store_true",
                    help="with --backward: time moe_layer_backward_saved on the state of a forward that kept its "
                         "activations, and that forward, and the two together")
    ap.add_argument("--replicas", type=int, default=-1, metavar="EXTRA",
                    help="time moe_layer_forward_replicated with EXTRA replicas dealt greedily to the most loaded "
                         "experts (counts from one plain forward of the same batch)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run a reference kernel of known traffic for hardware counters: read a buffer "
                         "of this many MiB and write its bitwise complement to another")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one layer call captured in a HIP graph instead of eager calls")
    ap.add_argument("--device-weights", action="store_true",
                    help="draw the expert weights on the device (torch's seeded generator, the same laws) "
                         "instead of on the host: for counter passes, whose figures do not depend on the "
                         "weights' values; implies --no-cpu-baseline")
    ap.add_argument("--counters-summary", metavar="DIR",
                    help="summarise the counter passes of --workload found under DIR/<workload>/<pass> and "
                         "print the summary (no GPU work)")
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


def sources_sha(stage: str) -> str:
    """sha256 over the kernel sources a stage's counters depend on."""
    h = hashlib.sha256()
    for name in STAGE_SOURCES[stage]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counters_file(workload: str) -> str:
    return os.path.join(PROFILES, f"moe_layer_{workload}_counters.txt")


def read_traffic(workload: str, stage: str):
    """HBM bytes per launch of a stage's kernel from the committed rocprofv3
    counter summary of this workload, if it was taken on the current kernel
    sources (else None)."""
    path = counters_file(workload)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_sha = re.search(rf"^{stage}_sources_sha256:\s*([0-9a-f]+)", txt, re.M)
    m_b = re.search(rf"^{stage}_hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt, re.M)
    if not (m_sha and m_b) or m_sha.group(1) != sources_sha(stage):
        return None
    return float(m_b.group(1))


def short_kernel_name(name: str) -> str:
    """'void moe::(anonymous namespace)::k<a, b>(args...)' -> 'k<a, b>'."""
    n = name.strip().strip('"')
    if n.startswith("void "):
        n = n[5:]
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):       # drop the argument list (the first '(' outside template brackets)
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not n.startswith("(anonymous", i):
            cut = i
            break
    n = n[:cut]
    return re.sub(r"^(?:[\w]+::|\(anonymous namespace\)::)+", "", n)


def stage_of_kernel(short: str):
    """The layer stage a forward kernel belongs to (None for the others)."""
    m = re.match(r"(gemm_\w+?)<(\w+)(?:, (\w+))?(?:, (\w+))?", short)
    if m:
        if m.group(2) == "true":
            return "gate_up"
        if m.group(1) == "gemm_bf16_dma_kernel" and m.group(4) == "true":
            return "router"                          # fp32-output score GEMM
        return "down"
    for prefix, stage in (("router_logits", "router"), ("route_kernel", "route"), ("scatter_rows", "scatter"),
                          ("slot_scatter", "scatter"), ("combine_kernel", "combine"), ("slots", "slots"), ("scan_kernel", "slots"),
                          ("tile_hist", "slots")):
        if short.startswith(prefix):
            return stage
    return None


def read_counter_csv(folder: str):
    """{short kernel name: {counter: [value per dispatch]}} from the
    *counter_collection.csv files rocprofv3 wrote under folder."""
    import csv
    import glob
    out = {}
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {folder}")
    for path in files:
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                k = short_kernel_name(row["Kernel_Name"])
                disp = row.get("Dispatch_Id") or row.get("Correlation_Id")
                cs = out.setdefault(k, {})
                cs.setdefault(row["Counter_Name"], {}).setdefault(disp, 0.0)
                cs[row["Counter_Name"]][disp] += float(row["Counter_Value"])
                try:   # the dispatch's duration (ns), as the profiled run timed it
                    cs.setdefault("duration_ns", {})[disp] = float(int(row["End_Timestamp"]) - int(row["Start_Timestamp"]))
                except (KeyError, ValueError):
                    pass
    return {k: {c: list(v.values()) for c, v in cs.items()} for k, cs in out.items()}


def counters_summary(root: str, workload: str) -> str:
    """Text summary of the counter passes of one workload (see PROFILE_PASSES)."""
    import numpy as np
    passes = {name: read_counter_csv(os.path.join(root, workload, name)) for name, _ in PROFILE_PASSES}
    probes = [k for k in passes["fetch"] if "bitwise_not" in k]
    if not probes:
        raise RuntimeError("no reference kernel (bitwise_not of the 1 GiB probe) in the fetch pass")
    copy = probes[0]
    f_fac = COPY_PROBE_KIB / np.mean(passes["fetch"][copy]["FETCH_SIZE"])
    w_fac = COPY_PROBE_KIB / np.mean(passes["write"][copy]["WRITE_SIZE"])
    lines = [f"rocprofv3 hardware counters of the MoE layer forward, workload {workload} (MI355X)", "",
             "Commands (from the repository root as $REPO, any output folder $OUT; one pass per run):"]
    for name, counters in PROFILE_PASSES:
        lines.append("  " + PROFILE_CMD.format(counters=counters, workload=workload, name=name))
    lines.append(f"  python $REPO/bench.py --workload {workload} --counters-summary $OUT")
    lines += ["", "HBM bytes: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by what each reads for the "
              f"reference kernel ({copy[:60]}..., 1 GiB read + 1 GiB written):",
              f"  FETCH_SIZE factor {f_fac:.5f}, WRITE_SIZE factor {w_fac:.5f}",
              "MFMA: SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 = executed bf16 matrix flops; MfmaUtil = matrix-core "
              "busy cycles summed over the 1024 SIMDs over (GRBM_GUI_ACTIVE x 1024), in %; wait = "
              "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (share of wave time waiting to issue); LDS bank = "
              "SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS (conflict cycles per LDS-active quad-cycle); "
              "GHz = GRBM_GUI_ACTIVE (summed over the 8 XCDs) / 8 / the profiled dispatch's duration, the "
              "clock the dispatch ran at; L2 hit = TCC_HIT / (TCC_HIT + TCC_MISS).", "",
              "Per dispatch (mean over the dispatches of the run):"]
    hdr = (f"{'kernel':62s} {'stage':8s} {'FETCH KiB':>11s} {'WRITE KiB':>11s} {'HBM bytes':>11s} "
           f"{'MFMA flop':>11s} {'MfmaUtil':>8s} {'wait':>6s} {'LDS bank':>8s} {'GHz':>5s} {'L2 hit':>7s}")
    lines.append(hdr)
    per_stage = {}
    for k in passes["fetch"]:
        def mean(p, c):
            v = passes[p].get(k, {}).get(c)
            return float(np.mean(v)) if v else float("nan")
        fk, wk = mean("fetch", "FETCH_SIZE"), mean("write", "WRITE_SIZE")
        hbm = (fk * f_fac + wk * w_fac) * 1024
        def ratio(a, b):
            return a / b if b > 0 else float("nan")
        mops, util = mean("mfma", "SQ_INSTS_VALU_MFMA_MOPS_BF16"), mean("mfma", "MfmaUtil")
        wait = ratio(mean("mfma", "SQ_WAIT_INST_ANY"), mean("mfma", "SQ_WAVE_CYCLES"))
        bank = ratio(mean("mfma", "SQ_LDS_BANK_CONFLICT"), mean("mfma", "SQ_ACTIVE_INST_LDS"))
        ghz = ratio(mean("mfma", "GRBM_GUI_ACTIVE") / 8, mean("mfma", "duration_ns"))
        hit, miss = mean("l2", "TCC_HIT_sum"), mean("l2", "TCC_MISS_sum")
        st = stage_of_kernel(k)
        lines.append(f"{k[:62]:62s} {st or '-':8s} {fk:11.1f} {wk:11.1f} {hbm:11.4e} {mops * 512:11.4e} "
                     f"{util:8.2f} {wait:6.3f} {bank:8.4f} {ghz:5.2f} "
                     f"{hit / (hit + miss) if hit + miss > 0 else float('nan'):7.3f}")
        if st:
            per_stage.setdefault(st, []).append(hbm)
    lines.append("")
    for st in ("gate_up", "down", "scatter", "combine"):
        if st in per_stage:
            lines.append(f"{st}_hbm_bytes_per_launch: {sum(per_stage[st]):.6e}")
            lines.append(f"{st}_sources_sha256: {sources_sha(st)}")
    return "\n".join(lines) + "\n"


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
    while len(times) < 3:    # median of three runs, or one run when a run takes over 10 s
        t0 = time.perf_counter()
        oracle.layer_forward(wl.x, wl.wr, lambda e: (host_w[0][e], host_w[1][e], host_w[2][e]), wl.T, wl.d,
                             wl.d_ff, wl.E, wl.k, wl.cf, wl.dtype, P=wl.P, bias=wl.bias_vec, tokens=tokens,
                             max_ranks=wl.max_ranks, replicas=replicas)
        times.append(time.perf_counter() - t0)
        if times[0] > 10.0:
            break
    dt = sorted(times)[len(times) // 2]
    runs = "median of 3 runs" if len(times) == 3 else "one run"
    return {"value": round(tokens.size / dt, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "host": host_cpu(),
            "sample": f"layer outputs of the first {tokens.size} of {wl.T} tokens (routing and slots of all "
                      f"{wl.T}; every touched expert's weights decoded), fp64 numpy, {runs}: {dt:.1f} s each "
                      f"({sum(times):.1f} s total)"}


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
    kept_state = None
    if args.saved:  # a forward that keeps its routing, buckets and activations
        C = moe.moe_capacity(T, E, k, cf)
        i32 = dict(dtype=torch.int32, device=dev)
        kept_state = {"out": torch.empty_like(x), "topk_idx": torch.empty((T, k), **i32),
                      "topk_w": torch.empty((T, k), dtype=torch.float32, device=dev),
                      "slot": torch.empty((T, k), **i32), "routed_count": torch.empty(E, **i32),
                      "kept_count": torch.empty(E, **i32), "send_count": torch.empty(P, **i32),
                      "totals": torch.empty(4, dtype=torch.int64, device=dev),
                      "buckets": torch.empty((E, C, d), dtype=x.dtype, device=dev)}
        for name in ("g", "u", "h"):
            kept_state[name] = torch.empty((E, C, d_ff), dtype=x.dtype, device=dev)
        fws_bytes = moe.moe_workspace_size(T, d, d_ff, E, k, cf, P, wl.dtype)
        fws = torch.empty(fws_bytes, dtype=torch.uint8, device=dev)

        def forward_keep():
            moe.moe_layer_forward(x, wr, bias, wg, wu, wd, T, d, d_ff, E, k, cf, P, wl.max_ranks, wl.dtype,
                                  kept_state["out"], kept_state, fws, fws_bytes, stream)

        forward_keep()

    def step():
        if kept_state is None:
            moe.moe_layer_backward(x, wr, bias, wg, wu, wd, dout, T, d, d_ff, E, k, cf, P, wl.max_ranks, wl.dtype,
                                   outs["dx"], outs["dW_router"], outs["d_bias"], outs["dW_gate"], outs["dW_up"],
                                   outs["dW_down"], ws, ws_bytes, stream)
        else:
            moe.moe_layer_backward_saved(x, wr, bias, wg, wu, wd, dout, T, d, d_ff, E, k, cf, P, wl.max_ranks,
                                         wl.dtype, kept_state, outs["dx"], outs["dW_router"], outs["d_bias"],
                                         outs["dW_gate"], outs["dW_up"], outs["dW_down"], ws, ws_bytes, stream)

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
    print(f"[bench] backward{' from the kept state' if args.saved else ''}: timed {args.steps} steps: "
          f"{wall * 1e3 / args.steps:.3f} ms/step wall, {gpu_ms:.3f} ms/step GPU", file=sys.stderr, flush=True)
    keep_ms = train_ms = None
    if args.saved:
        def timed(fn):
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for _ in range(args.steps):
                fn()
            torch.cuda.synchronize()
            return (time.perf_counter() - t1) * 1e3 / args.steps

        keep_ms = timed(forward_keep)
        train_ms = timed(lambda: (forward_keep(), step()))
        print(f"[bench] forward keeping its activations: {keep_ms:.3f} ms/step; with the backward from that "
              f"state: {train_ms:.3f} ms/step", file=sys.stderr, flush=True)
    # the kept copies (for the algorithmic flops) from the layer forward on the GPU
    if kept_state is None:
        kept_count = torch.empty(E, dtype=torch.int32, device=dev)
        fws_bytes = moe.moe_workspace_size(T, d, d_ff, E, k, cf, P, wl.dtype)
        fws = torch.empty(fws_bytes, dtype=torch.uint8, device=dev)
        moe.moe_layer_forward(x, wr, bias, wg, wu, wd, T, d, d_ff, E, k, cf, P, wl.max_ranks, wl.dtype,
                              torch.empty_like(x), {"kept_count": kept_count}, fws, fws_bytes, stream)
        del fws
    else:
        kept_count = kept_state["kept_count"]
    n_kept = int(kept_count.sum().item())
    algo = 12 * n_kept * d * d_ff  # dh, dX (two), dWd, dWg, dWu: 2 N d d_ff flop each
    done = algo + (0 if args.saved else 4 * n_kept * d * d_ff)  # plus the recomputed g and u
    tf = algo / gpu_ms / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # the fp64 backward costs about 3x the forward per token: at most 1024 tokens
        S = min(args.cpu_sample or 1024, T, 1024)
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
        "metric": "backward tokens/s per MoE layer (gradients of x, router and expert weights)"
                  + (" from the forward's kept state" if args.saved else ""),
        "value": round(T * args.steps / wall, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded Gaussian inputs, upstream gradient and random-init weights of the named shape)",
        "config": {"workload": wl.name, "T": T, "d": d, "E": E, "k": k, "d_ff": d_ff, "cf": cf, "P": P,
                   "max_ranks": wl.max_ranks, "N_kept": n_kept},
        "gpu_ms_per_step": round(gpu_ms, 4),
        "forward_keeping_state_ms": None if keep_ms is None else round(keep_ms, 4),
        "forward_and_backward_ms": None if train_ms is None else round(train_ms, 4),
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


def device_expert_weights(wl, torch, dev):
    """Expert weights drawn on the device with torch's generator, seeded from
    the workload's weight seed: N(0, 1/sqrt(fan_in)) rounded to the layer
    dtype, the laws of the host-drawn weights (not their bits)."""
    g = torch.Generator(device=dev)
    g.manual_seed(1000003 * (wl.weight_seed + 1))
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    out = []
    for shape, fan_in in (((wl.E, wl.d_ff, wl.d), wl.d), ((wl.E, wl.d_ff, wl.d), wl.d), ((wl.E, wl.d, wl.d_ff), wl.d_ff)):
        w = torch.empty(shape, dtype=dt, device=dev)
        per = max(1, (1 << 28) // (shape[1] * shape[2]))   # experts per draw: at most 1 GiB of fp32
        for e in range(0, wl.E, per):
            n = min(per, wl.E - e)
            w[e:e + n] = (torch.randn((n,) + shape[1:], generator=g, device=dev) * (fan_in ** -0.5)).to(dt)
        out.append(w)
    return tuple(out)


def main():
    args = parse()
    if args.counters_summary:
        sys.stdout.write(counters_summary(args.counters_summary, args.workload))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the layer here has no multi-GPU path (asked for --gpus "
              f"{args.gpus})", file=sys.stderr)
        sys.exit(2)
    if args.graph and args.backward:
        print("bench.py --graph times the forward only (a backward call can be captured as well; the graph tests "
              "do)", file=sys.stderr)
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

    if args.saved and not args.backward:
        sys.exit("--saved goes with --backward")
    if args.device_weights:
        if args.backward or args.replicas >= 0:
            sys.exit("--device-weights serves the plain forward's counter passes only")
        args.no_cpu_baseline = True
        host_w = None
        wg, wu, wd = device_expert_weights(wl, torch, dev)
    else:
        host_w = wl.all_expert_weights()
        if args.backward:
            run_backward(args, wl, moe, torch, np, dev, to_dev, host_w)
            return
        wg, wu, wd = (to_dev(a) for a in host_w)
    x, wr = to_dev(wl.x), to_dev(wl.wr)
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
        torch.bitwise_not(src, out=dst)   # one elementwise kernel: reads and writes every byte once
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    timed_step = step
    if args.graph:
        # one layer call captured once (the library allocates nothing and
        # never waits on the host), replayed on the same stream
        graph, cap = torch.cuda.CUDAGraph(), torch.cuda.Stream()
        cap.wait_stream(stream)
        eager_stream = stream
        with torch.cuda.graph(graph, stream=cap):
            stream = torch.cuda.current_stream()
            step()
        stream = eager_stream
        torch.cuda.synchronize()
        timed_step = graph.replay
        for _ in range(args.warmup):
            timed_step()
        torch.cuda.synchronize()

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        timed_step()
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
                # a stage that launched nothing recorded no events: no time
                acc += [evs[2 * i].elapsed_time(evs[2 * i + 1]) if moe.moe_stage_ran(i) else 0.0
                        for i in range(len(moe.STAGES))]
                layer_ms.append(evs[0].elapsed_time(evs[-1]))
        finally:
            moe.moe_set_stage_events(None)
        del flush
        for i, name in enumerate(moe.STAGES):
            ms = acc[i] / args.steps
            w = work[name]
            # a stage with no kernels in it gets no rate
            timed = ms > 1e-3
            s = {"ms": round(ms, 5), "algo_bytes": int(w["bytes"]),
                 "GB_per_s": round(w["bytes"] / ms / 1e6, 1) if timed else None,
                 "hbm_frac": round(w["bytes"] / ms / 1e6 / PEAK_HBM_GBS, 4) if timed else None}
            if w["flops"]:
                s["TFLOP_per_s"] = round(w["flops"] / ms / 1e9, 1) if timed else None
                s["mfma_frac"] = round(w["flops"] / ms / 1e9 / PEAK_TFLOPS[wl.dtype], 4) if timed else None
            stages[name] = s
            print(f"[bench] stage {name:8s} {ms:8.4f} ms  " + " ".join(f"{a}={b}" for a, b in s.items()
                                                                       if a != "ms"), file=sys.stderr, flush=True)

    roofline = None
    if stages:
        dom = max(stages, key=lambda n: stages[n]["ms"])
        w, s = work[dom], stages[dom]
        traffic = read_traffic(wl.name, dom) if (dom in STAGE_SOURCES and reps is None) else None
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
        sample = args.cpu_sample if args.cpu_sample is not None else CPU_SAMPLE.get(wl.name, T)
        print(f"[bench] timing the CPU oracle on {min(sample, T)} tokens", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, host_w, sample, reps)

    metric = METRIC if reps is None else METRIC + " (hot experts replicated)"
    line = {
        "metric": metric, "value": round(T * args.steps / wall, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded Gaussian inputs and random-init weights of the named shape)",
        "config": {"workload": wl.name, "T": T, "d": d, "E": E, "k": k, "d_ff": d_ff, "cf": cf, "P": P,
                   "max_ranks": wl.max_ranks, "C": C, "N_kept": n_kept, "touched_experts": touched,
                   "dropped": totals[0], "launch": "hip_graph_replay" if args.graph else "eager", **repl_cfg},
        "gpu_ms_per_step": round(gpu_ms, 4),
        "assignments_per_s": round(T * k * args.steps / wall, 1),
        "layer_ms_cold_median": layer_cold,
        "stage_timing": None if not stages else (
            f"HIP events around each stage, mean of {args.steps} steps, each after a {args.flush_mib} MiB read "
            "that leaves none of the layer's data in L2 or the Infinity Cache"),
        "grouped_gemm_mfma_frac": None if not stages else round(
            (work["gate_up"]["flops"] + work["down"]["flops"]) /
            ((stages["gate_up"]["ms"] + stages["down"]["ms"]) * 1e9) / PEAK_TFLOPS[wl.dtype], 4),
        # the permutation (scan, capacity, slots and drop mask, scatter) over its
        # whole span; the scatter kernel alone beside it
        "permute_hbm_frac": None if not stages else round(
            (work["slots"]["bytes"] + work["scatter"]["bytes"]) /
            ((stages["slots"]["ms"] + stages["scatter"]["ms"]) * 1e6) / PEAK_HBM_GBS, 4),
        "scatter_hbm_frac": None if not stages else stages["scatter"]["hbm_frac"],
        "combine_hbm_frac": None if not stages else stages["combine"]["hbm_frac"],
        "stages": stages, "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
