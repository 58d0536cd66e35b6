#!/usr/bin/env python3
"""KDA chunked prefill throughput on one MI355X.

A step is one kda_fwd call over the whole workload (every token of every head,
final state included) with the inputs already resident in HBM. Default
workload: B=1, T=8192, H=96, K=V=128, bf16 q/k/v, fp32 g/beta/state, h0 = 0,
returns hT (the shape the H20 benchmark table on the toolarium.ru FlashKDA page
quotes first, section "Что показывают H20-бенчмарки"). Seeded synthetic inputs.

Prints one JSON line with tokens/s, the HBM roofline of the fused kernel
(algorithmic bytes / measured launch time) and the CPU oracle's throughput on
this host as a baseline.
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
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0
BYTES_PER_TOKEN_HEAD = 3 * 256 + 512 + 4 + 512   # q, k, v bf16 + g fp32 + beta + o fp32
STATE_BYTES = 128 * 128 * 4                        # one (sequence, head) state, fp32
# Chunked form at C = 64: 2*(3KV + K(C-1)/2 + (C+1)/2*(2K+2V) + C^2/6) flop per
# token-head with K = V = 128 (inter-chunk products, intra-chunk triangles, solve).
FLOPS_PER_TOKEN_HEAD = 141013

# Algorithmic bytes of each stage of the staged path (fp32 intermediates,
# 32-token chunks), per token-head: each tensor read or written once.
STAGE_BYTES = {
    "a1_gate_scan": 512 + 512 + 16,                      # g in; Gamma, gamma_last out
    "a2_intra": 768 + 512 + 4 + 4 * 512 + 128,           # q, k, v, Gamma, beta in; W, U, Kt, Qg, M out
    "a3_recurrence": 3 * 512 + 16 + 2048 + 512,          # W, U, Kt, gamma_last in; h_c, Delta out
    "a4_output": 512 + 2048 + 128 + 512 + 512,           # Qg, h_c, M, Delta in; o out
}


def alg_bytes(cfg) -> int:
    per_state = STATE_BYTES * cfg.N * cfg.H
    return cfg.token_heads * BYTES_PER_TOKEN_HEAD + per_state * (1 + (1 if cfg.h0 else 0))


def kernel_source_hash() -> str:
    """Hash of the sources the fused kernel is compiled from (its file and the
    device helpers it includes), so a counter summary is tied to that kernel."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_63_amd", "csrc")
    for f in ("kda_fused_pipe.hip", "kda_device.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"kda_fwd_pipe_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*(\w+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_hash or not m_b or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_b.group(1))


def host_description() -> dict:
    """The CPU the oracle baseline ran on: model name, logical CPUs and the
    OpenMP thread setting."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "sched_affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def calib_copy(args):
    """One device-to-device copy of --calib-copy-mb MiB, so that a counter pass
    over this run can scale its byte counters by a transfer of known size."""
    if not args.calib_copy_mb:
        return
    import torch
    nbytes = args.calib_copy_mb << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] calibration copy of {nbytes} bytes done", file=sys.stderr, flush=True)


def copy_bandwidth(nbytes: int = 1 << 30, reps: int = 20):
    """Device-to-device copy bandwidth on this GPU (bytes read plus bytes written
    per second, GB/s), timed with events over `reps` copies of `nbytes` after
    three untimed ones: the practical HBM ceiling the roofline fraction is also
    quoted against."""
    import torch
    try:
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
    except RuntimeError:
        return None
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    stream = torch.cuda.current_stream()
    a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    b_.record(stream)
    torch.cuda.synchronize()
    sec = a_.elapsed_time(b_) / 1e3 / reps
    del src, dst
    return 2 * nbytes / sec / 1e9


def bench_decode(args):
    """In-place decode steps: N sequences x 96 heads, one token each per step."""
    import numpy as np
    import torch
    import workloads as W
    import gated_delta_rule_63_amd as kda

    N, H = args.decode, W.CONFIGS["T8192_H96"].H
    cfg = W.variant("T8192_H96", B=N, T=1, H=H, h0=True, name=f"decode N={N}")
    inp = W.make_inputs(cfg, args.seed)
    dev = torch.device("cuda:0")
    cvt = lambda x: torch.from_numpy(W.bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = cvt(inp.q), cvt(inp.k), cvt(inp.v)
    g, beta = torch.from_numpy(inp.g).to(dev), torch.from_numpy(inp.beta).to(dev)
    state = torch.from_numpy(inp.h0).to(dev)
    o = torch.empty((N, 1, H, 128), dtype=torch.float32, device=dev)
    one = lambda: kda.decode_step(q, k, v, g, beta, state=state, out=o, in_place=True)
    step = one
    G = args.graph
    if G:
        # G steps captured once and replayed: one graph launch per G steps, so
        # the per-call cost of the binding and the launch is paid once per G
        one()
        torch.cuda.synchronize()
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                for _ in range(G):
                    one()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        step = graph.replay
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps / max(G, 1)
    per_head = 3 * 256 + 512 + 4 + 512 + 2 * STATE_BYTES
    bytes_ = N * H * per_head
    achieved = bytes_ / (ms / 1e3) / 1e9
    calib_copy(args)
    print(json.dumps({
        "metric": f"KDA decode tokens/s (N={N} sequences, H={H}, D=128, bf16, state in place)",
        "value": N / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"decode: {N} sequences x {H} heads, one token each, fp32 state read and written"
                               + (f", {G} steps per HIP graph launch" if G else ""),
                   "global_batch": N, "seq_len": 1, "heads": H, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "kda_decode_kernel",
                     "alg_bytes_per_launch": bytes_},
    }))


def bench_gdn(args):
    """Gated DeltaNet (one gate per token-head) at a prefill workload's shape."""
    import numpy as np
    import torch
    import workloads as W
    import gated_delta_rule_63_amd as kda

    cfg = W.variant(args.config, gate="scalar", name=args.config + " scalar gate")
    inp = W.make_inputs(cfg, args.seed)
    dev = torch.device("cuda:0")
    cvt = lambda x: torch.from_numpy(W.bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = cvt(inp.q), cvt(inp.k), cvt(inp.v)
    gs = torch.from_numpy(inp.g_scalar()).to(dev)
    beta = torch.from_numpy(inp.beta).to(dev)
    cu = torch.from_numpy(inp.cu_seqlens).to(dev) if inp.cu_seqlens is not None else None
    h0 = torch.from_numpy(inp.h0).to(dev) if inp.h0 is not None else None
    o = torch.empty((cfg.B, cfg.T, cfg.H, 128), dtype=torch.float32, device=dev)
    hT = torch.empty((cfg.N, cfg.H, 128, 128), dtype=torch.float32, device=dev)
    step = lambda: kda.gdn_fwd(q, k, v, gs, beta, cu_seqlens=cu, initial_state=h0, out=o, final_state=hT)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    per_token_head = 3 * 256 + 4 + 4 + 512          # q, k, v bf16, g and beta fp32, o fp32
    bytes_ = cfg.token_heads * per_token_head + STATE_BYTES * cfg.N * cfg.H * (1 + (1 if cfg.h0 else 0))
    achieved = bytes_ / (ms / 1e3) / 1e9
    calib_copy(args)
    print(json.dumps({
        "metric": f"Gated DeltaNet prefill tokens/s ({cfg.name}, T={cfg.T}, H={cfg.H}, D=128 bf16)",
        "value": cfg.B * cfg.T / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: one gate per (token, head)", "global_batch": cfg.B,
                   "seq_len": cfg.T, "heads": cfg.H, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "kda_fwd_pipe (scalar gate)",
                     "alg_bytes_per_launch": bytes_},
    }))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", default="T8192_H96")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--protocol-repeats", type=int, default=5,
                    help="extra repeats of --steps iterations (the pages' 30/200/5 protocol)")
    ap.add_argument("--path", choices=["fused", "staged"], default="fused",
                    help="fused: kda_fwd (the hot path); staged: kda_fwd_staged (five kernels)")
    ap.add_argument("--kernel", choices=["auto", "pipe", "serial", "chunk16", "two_pass"], default="auto",
                    help="fused path: run this one forward kernel (kda_fwd_kernel); chunk16 is the "
                         "16-token-chunk ablation of the serial kernel, two_pass the two-kernel form "
                         "of the pipelined one (its workspace allocated once, outside the timed steps)")
    ap.add_argument("--stages", action="store_true", help="also time each staged-path kernel on its own")
    ap.add_argument("--decode", type=int, default=0, metavar="N",
                    help="time the in-place decode step for N sequences (H = 96) instead of the prefill")
    ap.add_argument("--graph", type=int, default=0, metavar="G",
                    help="with --decode: capture G decode steps in one HIP graph and time its replays")
    ap.add_argument("--gdn", action="store_true",
                    help="time the scalar-gate (Gated DeltaNet) forward at --config's shape instead")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run one device-to-device copy of this many MiB at the end (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only (--gpus must be 1); the kernels shard by head across GPUs without communication, which is not implemented here",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    if args.gdn:
        bench_gdn(args)
        return
    if args.decode:
        bench_decode(args)
        return

    import numpy as np
    import torch
    import workloads as W
    import gated_delta_rule_63_amd as kda

    cfg = W.CONFIGS[args.config]
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    log(f"[bench] generating {cfg.name} inputs (seed {args.seed})")
    inp = W.make_inputs(cfg, args.seed)
    dev = torch.device("cuda:0")
    if cfg.dtype == "bf16":
        cvt = lambda x: torch.from_numpy(W.bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        cvt = lambda x: torch.from_numpy(x).to(dev)
    q, k, v = cvt(inp.q), cvt(inp.k), cvt(inp.v)
    g, beta = torch.from_numpy(inp.g).to(dev), torch.from_numpy(inp.beta).to(dev)
    cu = torch.from_numpy(inp.cu_seqlens).to(dev) if inp.cu_seqlens is not None else None
    h0 = torch.from_numpy(inp.h0).to(dev) if inp.h0 is not None else None
    o = torch.empty((cfg.B, cfg.T, cfg.H, 128), dtype=torch.float32, device=dev)
    hT = torch.empty((cfg.N, cfg.H, 128, 128), dtype=torch.float32, device=dev)

    if args.path == "fused":
        # the workspace the forward would otherwise allocate, once, outside the timed steps
        nws = kda.kernel_workspace_size(q, args.kernel, cu) if args.kernel != "auto" else kda.fwd_workspace_size(q, cu)
        ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None

        def step():
            kda.fwd(q, k, v, g, beta, cu_seqlens=cu, initial_state=h0, out=o, final_state=hT, kernel=args.kernel,
                    workspace=ws)
    else:
        st = kda.Staged(q, k, v, g, beta, cu_seqlens=cu, initial_state=h0)

        def step():
            st.chunk_map()
            st.gate_scan()
            st.intra()
            st.recurrence(hT)
            st.output(o)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps

    # the pages' protocol: repeats of `steps` iterations, median of per-iteration means
    reps = []
    for _ in range(args.protocol_repeats):
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        for _ in range(args.steps):
            step()
        b_.record(stream)
        torch.cuda.synchronize()
        reps.append(a_.elapsed_time(b_) / args.steps)

    stage_times = None
    if args.stages:
        st = st if args.path == "staged" else kda.Staged(q, k, v, g, beta, cu_seqlens=cu, initial_state=h0)
        st.chunk_map()
        st.gate_scan()
        st.intra()
        st.recurrence(hT)
        torch.cuda.synchronize()
        stage_times = {}
        for name, fn in (("a0_chunk_map", st.chunk_map), ("a1_gate_scan", st.gate_scan), ("a2_intra", st.intra),
                         ("a3_recurrence", lambda: st.recurrence(hT)), ("a4_output", lambda: st.output(o))):
            n_it = max(3, args.steps // 10)
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            for _ in range(n_it):
                fn()
            b_.record(stream)
            torch.cuda.synchronize()
            t_ms = a_.elapsed_time(b_) / n_it
            entry = {"ms": t_ms}
            if name in STAGE_BYTES:
                gbs = cfg.token_heads * STAGE_BYTES[name] / (t_ms / 1e3) / 1e9
                entry.update({"alg_bytes_per_token_head": STAGE_BYTES[name], "achieved_GBs": gbs,
                              "frac_hbm": gbs / HBM_PEAK_GBS})
            stage_times[name] = entry
        log(f"[bench] stages: {stage_times}")

    calib_copy(args)
    copy_gbs = copy_bandwidth()

    tokens = cfg.B * cfg.T
    value = tokens / (ms / 1e3)
    bytes_ = alg_bytes(cfg)
    achieved = bytes_ / (ms / 1e3) / 1e9
    flops = cfg.token_heads * FLOPS_PER_TOKEN_HEAD
    if args.path == "staged":
        kname = "staged path (5 kernels)"
    elif args.kernel == "auto":
        kname = "kda_fwd_pipe" if cfg.dtype == "bf16" else "kda_fwd_fused (serial)"
    else:
        kname = {"pipe": "kda_fwd_pipe", "serial": "kda_fwd_fused (serial)", "chunk16": "kda_fwd_chunk16",
                 "two_pass": "kda_prep_pipe + kda_recur_pipe"}[args.kernel]
    # the counter summary covers the pipelined kernel as kda_fwd runs it
    traffic = traffic_from_profile(cfg.name) if (kname == "kda_fwd_pipe" and args.kernel == "auto") else None

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("[bench] CPU oracle baseline (fp64 recurrence, whole workload, repeated for >= 10 s)")
        runs, t0 = 0, time.perf_counter()
        while True:
            oracle.kda_ref_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, cu_seqlens=inp.cu_seqlens, h0=inp.h0)
            runs += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0 or runs >= 50:
                break
        cpu = {"value": tokens * runs / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
               "sample": f"the whole {cfg.name} workload ({cfg.token_heads} token-heads) {runs} times, {dt:.1f} s",
               "host": host_description()}
        cpu["gpu_over_oracle"] = value / cpu["value"]

    desc = f"{cfg.name}: B={cfg.B} T={cfg.T} H={cfg.H} K=V=128 {cfg.dtype} q/k/v, fp32 g/beta/state"
    if cfg.seq_lens:
        desc += f", varlen {list(cfg.seq_lens)}"
    desc += ", h0 given" if cfg.h0 else ", h0 = 0"
    out = {
        "metric": "KDA prefill tokens/s (T=8192,H=96,D=128 bf16) + % of MFMA/HBM roofline",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": desc + ("" if args.kernel == "auto" else f", kernel {args.kernel}"),
                   "global_batch": cfg.B, "seq_len": cfg.T, "heads": cfg.H, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kname, "alg_bytes_per_launch": bytes_,
                     "copy_GBs": copy_gbs, "frac_of_copy": achieved / copy_gbs if copy_gbs else None},
        "mfma": {"achieved": flops / (ms / 1e3) / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": flops / (ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
        "protocol": {"repeats": len(reps), "iters": args.steps, "median_ms": float(np.median(reps)) if reps else None,
                     "min_ms": min(reps) if reps else None, "max_ms": max(reps) if reps else None},
        "path": args.path,
        "stages": stage_times,
        "wall_s_timed_region": wall,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
