#!/usr/bin/env python3
"""Throughput of Linformer attention on one MI355X: tokens/s for one non-causal encoder layer at
B8 H12 n4096 d64 k256 bf16 with unshared per-head E, F and padded lengths in [2048, 4096].

A step is one linformer_forward call (sequence projection, then compressed attention) over the
whole batch, inputs already resident in device memory.  Input replicas are rotated so that
consecutive steps do not find their inputs in the 256 MB last-level cache.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Linformer attention tokens/s at n=4096,k=256 bf16; % of MFMA/HBM roofline"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "efficient_transformer_attention_seq_amd", "csrc")
# the source files each kernel's code comes from (a recorded time or traffic is valid only while
# their hash is unchanged)
KERNEL_SOURCES = {"attend": ("attend_bf16.hip", "attend_core.h", "lf_device.h"),
                  "project": ("proj_bf16.hip", "lf_device.h"),
                  "fused": ("fused_bf16.hip", "attend_core.h", "lf_device.h"),
                  "attend_f32": ("f32_path.hip", "lf_device.h")}
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def uses_fused(wl, conv: bool) -> bool:
    """Whether linformer_forward runs this workload as the one-launch fused kernel: the library's
    rule (bf16, n <= 1024, k of 128 or 256, one matrix for keys and values)."""
    return (not conv and wl.dtype == 1 and wl.n <= 1024 and wl.k in (128, 256)
            and not wl.separate_f and os.environ.get("LINFORMER_FUSED", "1") != "0")


def step_algorithmic(wl, conv: bool = False):
    """(bytes, flops) of one forward step as the scope table counts the method's work: Q, K, V
    read and O written once over the padded length, each distinct E/F matrix read once (the
    window weights of the convolution compression are negligible); 8 n k d flops per (b, h).
    The Kbar/Vbar intermediates are not counted."""
    B, H, n, d, k = wl.batch, wl.heads, wl.n, wl.d, wl.k
    eb = 2 if wl.dtype == 1 else 4
    n_mats = wl.e_heads * (2 if wl.separate_f else 1)
    byts = 4 * B * H * n * d * eb + (0 if conv else n_mats * k * n * eb)
    flops = B * H * (4.0 * n * k * d + (4.0 * n * d if conv else 4.0 * n * k * d))
    return byts, flops


def source_hashes() -> dict:
    """sha256/16 of every kernel and host source of the library and of its header, and one hash
    over all of them: the key that ties a recorded number to the code that produced it."""
    files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp", ".h")))
    out, h = {}, hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            data = fh.read()
        out[f] = hashlib.sha256(data).hexdigest()[:16]
        h.update(data)
    with open(os.path.join(ROOT, "include", "linformer.h"), "rb") as fh:
        data = fh.read()
    out["linformer.h"] = hashlib.sha256(data).hexdigest()[:16]
    h.update(data)
    out["all"] = h.hexdigest()[:16]
    return out


def rocprof_us(kernel: str, workload: str):
    """Average kernel duration (us) from the committed rocprofv3 kernel trace of this workload,
    if it was taken on the current kernel source (profiles/kernel_times.txt); else None.

    kernel_times.txt lines: <kernel> <workload> <source sha256, 16 hex> <average ns>
    """
    path = os.path.join(PROFILES, "kernel_times.txt")
    if not os.path.exists(path):
        return None
    sha = source_hash(kernel)
    with open(path) as f:
        for line in f:
            parts = line.split()
            if line.startswith("#") or len(parts) != 4:
                continue
            if parts[0] == kernel and parts[1] == workload and parts[2] == sha:
                return float(parts[3]) / 1e3
    return None


def traffic_bytes(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE/WRITE_SIZE (copy-calibrated), from
    profiles/traffic.txt, if they were taken on the current kernel source; else None.

    traffic.txt lines: <kernel> <workload> <source sha256, 16 hex> <fetch bytes> <write bytes>
    """
    path = os.path.join(PROFILES, "traffic.txt")
    if not os.path.exists(path):
        return None
    sha = source_hash(kernel)
    with open(path) as f:
        for line in f:
            if line.startswith("#"):
                continue
            parts = line.split()
            if len(parts) == 5 and parts[0] == kernel and parts[1] == workload and parts[2] == sha:
                return int(parts[3]) + int(parts[4])
    return None


def algorithmic(wl, kernel: str, conv: bool = False):
    """(bytes, flops) per launch as the method's work is counted in the scope table: over the
    padded length n (tokens = B n), in the workload's storage type (bf16, or fp32).

    Per token and head: project reads K and V (2 d 2 B = 256 B) plus its share of each distinct
    E/F matrix (read once), and does 4 k d flops (Kbar and Vbar); attend reads Q and writes O
    (256 B) and does 4 k d flops (scores and weighted sum).  Kbar/Vbar (B H k d, bf16) are counted
    once as the projection's output and once as the attention's input.  The kernels skip the
    rows past each length, so their real traffic (profiles/traffic.txt) is lower on padded
    workloads; the storage format's extra Kbar residual bytes are not counted either.
    """
    B, H, n, d, k = wl.batch, wl.heads, wl.n, wl.d, wl.k
    bh = B * H
    eb = 2 if wl.dtype == 1 else 4
    kv = 2 * bh * k * d * eb
    flops = 4.0 * bh * n * k * d
    if kernel == "project":
        if conv:   # one multiply-add per key / value element
            flops = 4.0 * bh * n * d
        n_mats = wl.e_heads * (2 if wl.separate_f else 1)
        # the convolution compression reads window weights (negligible) instead of E and F
        byts = 2 * bh * n * d * eb + (0 if conv else n_mats * k * n * eb) + kv
    else:
        byts = 2 * bh * n * d * eb + kv
    return byts, flops


def cpu_baseline(inp, min_s: float = 10.0, budget_s: float = 30.0):
    """The float64 oracle, as it stands, on the host cores: whole passes over the workload,
    repeated until at least `min_s` seconds of work (or, if one pass is slower than `budget_s`,
    the first batch items that fit that budget)."""
    import numpy as np
    from oracle import linformer_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    wl = inp.wl
    pairs_all = [(b, h) for b in range(wl.batch) for h in range(wl.heads)]
    # time one batch item first, then as many as fit the budget
    t0 = time.perf_counter()
    orc.forward(inp.Q, inp.K, inp.V, inp.E, inp.F, wl.share, inp.lengths,
                pairs=pairs_all[:wl.heads])
    t1 = time.perf_counter() - t0
    nb = max(1, min(wl.batch, int(budget_s / max(t1, 1e-6))))
    passes = 1
    if nb == wl.batch:
        # whole passes: as many as make up min_s
        t0 = time.perf_counter()
        orc.forward(inp.Q, inp.K, inp.V, inp.E, inp.F, wl.share, inp.lengths, pairs=pairs_all)
        one = time.perf_counter() - t0
        passes = max(1, int(np.ceil(min_s / max(one, 1e-6))))
        t0 = time.perf_counter()
        for _ in range(passes):
            orc.forward(inp.Q, inp.K, inp.V, inp.E, inp.F, wl.share, inp.lengths, pairs=pairs_all)
        dt = time.perf_counter() - t0
    elif nb > 1:
        t0 = time.perf_counter()
        orc.forward(inp.Q, inp.K, inp.V, inp.E, inp.F, wl.share, inp.lengths,
                    pairs=pairs_all[:nb * wl.heads])
        dt = time.perf_counter() - t0
    else:
        nb, dt = 1, t1
    tokens = passes * nb * wl.n
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    del np
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{passes} pass(es) over {nb} of {wl.batch} batch items "
                      f"({nb * wl.heads} (b,h) slices each), full n={wl.n}, float64 numpy, "
                      f"{dt:.2f} s on {cpu}",
            "seconds": dt}


def copy_ceiling(torch, mib: int = 512, iters: int = 10) -> float:
    """Read + write GB/s of a plain device copy of `mib` MiB: the practical HBM ceiling."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    sec = a.elapsed_time(b) / 1e3 / iters
    del src, dst
    return 2 * (mib << 20) / sec / 1e9


def run_sweep(L, synth, torch, np):
    """Forward time against n at B1 H12, k = 128 and 256, layerwise E = F, bf16, no padding, with
    the O(n^2) comparator up to n = 16384.  Prints one JSON line with the table."""
    rows = []
    for k in (128, 256):
        for n in (512, 1024, 2048, 4096, 8192, 16384, 32768, 65536):
            inp = synth.random_inputs(1, 12, n, 64, k, synth.DT_BF16, synth.SHARE_LAYERWISE,
                                      seed=n + k)
            td = torch.bfloat16
            dev = lambda x: torch.from_numpy(x).to(td).cuda()
            Q, K, V, E = dev(inp.Q), dev(inp.K), dev(inp.V), dev(inp.E)
            p = L.problem(1, 12, n, 64, k, synth.DT_BF16, synth.SHARE_LAYERWISE, 0.0)
            O = torch.empty(1, 12, n, 64, dtype=td, device="cuda")
            wsb = L.linformer_workspace_size(p)
            ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")

            def fwd():
                L.linformer_forward(p, Q, K, V, E, None, None, O, ws, wsb)

            def dense():
                L.attention_dense_forward(p, Q, K, V, None, O)

            def timed(fn, iters):
                for _ in range(3):
                    fn()
                torch.cuda.synchronize()
                ts = []
                for _ in range(iters):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record()
                    fn()
                    b.record()
                    b.synchronize()
                    ts.append(a.elapsed_time(b) * 1e3)
                return float(np.median(ts))

            us = timed(fwd, 20)
            row = {"k": k, "n": n, "linformer_us": round(us, 2),
                   "tokens_per_s": round(n / (us * 1e-6), 1)}
            if n <= 16384:
                dus = timed(dense, 10)
                row["dense_us"] = round(dus, 2)
                row["speedup"] = round(dus / us, 2)
            rows.append(row)
            log(f"k={k:4d} n={n:6d}: linformer {us:9.1f} us" +
                (f", dense {row['dense_us']:9.1f} us, {row['speedup']:.2f}x" if "dense_us" in row else ""))
            del Q, K, V, E, O, ws
    print(json.dumps({"sweep": rows, "config": {"batch": 1, "heads": 12, "head_dim": 64,
                                                "share": "layerwise", "dtype": "bf16"},
                      "time_basis": "median of per-call HIP event pairs on the launch stream",
                      "source_sha": source_hashes(),
                      "command": "python bench.py " + " ".join(sys.argv[1:])}), flush=True)


def stack_flops(wl) -> float:
    """Method-equivalent matrix flops of one pass of the encoder attention stack, counted as the
    definition states it: per layer the input projection (2 T d_model 3 d_model), Linformer
    attention (8 n k d per head and batch item: Kbar, Vbar, scores, weighted sum) and the output
    projection (2 T d_model^2), T = B n tokens."""
    T, dm = wl.batch * wl.n, wl.d_model
    per_layer = 2.0 * T * dm * 3 * dm + 2.0 * T * dm * dm + 8.0 * wl.batch * wl.heads * wl.n * wl.k * 64
    return wl.layers * per_layer


def stack_executed_flops(wl) -> float:
    """bf16 matrix flops linformer_stack_forward executes per pass (the keys and values are
    formed as (E X) W^T over the k projected rows, not as E (X W^T)): per layer the query
    projection (2 T d_model^2), the sequence projection of the layer input E X (2 B k n d_model),
    the projected keys and values (2 B k d_model 2 d_model), the scores and weighted sum
    (4 n k d per head and batch item) and the output projection (2 T d_model^2).  The residual
    product of the scores (e4m3, at twice the bf16 rate) is not counted."""
    T, dm, B, k, n = wl.batch * wl.n, wl.d_model, wl.batch, wl.k, wl.n
    per_layer = (2.0 * T * dm * dm + 2.0 * B * k * n * dm + 2.0 * B * k * dm * 2 * dm +
                 4.0 * B * wl.heads * n * k * 64 + 2.0 * T * dm * dm)
    return wl.layers * per_layer


def stack_cpu_baseline(si, min_s: float = 10.0):
    """The float64 oracle of the stack on the host cores: batch items through every layer, one
    at a time, until at least `min_s` seconds of work."""
    from oracle import linformer_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    wl = si.wl
    t0 = time.perf_counter()
    items = 0
    while True:
        b = items % wl.batch
        orc.stack_forward(si.X[b:b + 1], si.Wqkv, si.Wo, si.E, wl.heads)
        items += 1
        dt = time.perf_counter() - t0
        if dt >= min_s:
            break
    return {"value": items * wl.n / dt, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{items} batch items of {wl.n} tokens (cycling over the {wl.batch}) "
                      f"through all {wl.layers} layers, float64 numpy, {dt:.2f} s",
            "seconds": dt}


def run_stack_bench(args, L, synth, torch, np):
    """One step = linformer_stack_forward over the whole batch (every layer)."""
    wl = synth.STACK_WORKLOADS[args.workload]
    log(f"workload {wl}")
    si = synth.make_stack_inputs(wl)
    s = L.stack(wl.batch, wl.n, wl.d_model, wl.heads, wl.k, wl.layers, False, 0.0)
    bf = torch.bfloat16

    def dev(x):
        return torch.from_numpy(x).to(bf).cuda()

    Wq, Wo, E = dev(si.Wqkv), dev(si.Wo), dev(si.E)
    if args.replicas <= 0:   # the activations are the only per-step input; weights stay resident
        args.replicas = max(2, -(-(1 << 30) // si.X.size // 2))
    Xs = [dev(si.X) for _ in range(args.replicas)]
    Y = torch.empty(wl.batch, wl.n, wl.d_model, dtype=bf, device="cuda")
    wsb = L.linformer_stack_workspace_size(s)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        L.linformer_stack_forward(s, Xs[i % len(Xs)], Wq, Wo, E, None, Y, ws, wsb, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = ev0.elapsed_time(ev1) / args.steps
    tokens = wl.batch * wl.n
    flops = stack_executed_flops(wl)
    tflops = flops / (ms * 1e-3) / 1e12
    eq_flops = stack_flops(wl)
    log(f"stack: {ms * 1e3:.1f} us/step ({tokens / (ms / 1e3):.3e} tokens/s), "
        f"{tflops:.1f} TFLOP/s executed ({flops / 1e9:.0f} GFLOP per step; method-equivalent "
        f"{eq_flops / 1e9:.0f} GFLOP)")
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on the host cores ...")
        cpu = stack_cpu_baseline(si)
        log(f"oracle: {cpu['value']:.3e} tokens/s ({cpu['sample']})")
    out = {
        "metric": "Linformer encoder attention stack tokens/s (12 layers); % of MFMA roofline",
        "value": round(tokens / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.n,
                   "d_model": wl.d_model, "heads": wl.heads, "k": wl.k, "layers": wl.layers,
                   "share": "layerwise", "replicas": args.replicas},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": "whole step (projections, attention)",
                     "executed_flops": flops,
                     "method_equivalent_flops": eq_flops,
                     "method_equivalent_frac": round(eq_flops / (ms * 1e-3) / 1e12 /
                                                     PEAK_BF16_TFLOPS, 4)},
        "time_basis": "HIP events around the timed back-to-back stack calls on the launch stream",
        "source_sha": source_hashes(),
        "command": "python bench.py " + " ".join(sys.argv[1:]),
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(0),
        "wall_s": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


def library_allocation(torch, fn, warm: int = 2, calls: int = 3) -> int:
    """Change of the device's free memory (hipMemGetInfo, through torch.cuda.mem_get_info) over
    `calls` calls of `fn` after `warm` warm-up calls: the device memory the library itself takes.
    Torch allocates nothing in between, so only the library or the runtime could move it."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(calls):
        fn()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    return int(free0 - free1)


def standard_attention_bytes(torch, B, H, n, d):
    """Peak device bytes, beyond its inputs and output, of standard softmax attention written
    with plain torch operations as the pages' baseline computes it: the n x n scores in fp32,
    their softmax, the probabilities in bf16, then the weighted sum of V (torch's allocator
    sees every one of these tensors)."""
    bf = torch.bfloat16
    Q = torch.randn(B, H, n, d, device="cuda").to(bf)
    K = torch.randn(B, H, n, d, device="cuda").to(bf)
    V = torch.randn(B, H, n, d, device="cuda").to(bf)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    # fp32 operands (a transposed bf16 right operand of a batched product is avoided)
    Kt = K.float().transpose(-1, -2).contiguous()
    S = torch.matmul(Q.float(), Kt) * (1.0 / d ** 0.5)
    del Kt
    P = torch.softmax(S, dim=-1).to(bf)
    del S
    O = torch.matmul(P, V)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    del Q, K, V, P, O
    torch.cuda.empty_cache()
    return int(peak)


def run_memory(L, synth, torch, np):
    """Device memory of one attention layer per batch item, Linformer against standard attention,
    and the largest batch that fits on this GPU (H = 12, d = 64, bf16, layerwise E = F) -- the
    pages' memory figure is a ratio of such largest batches.

    Measured: (1) what liblinformer itself allocates on the device -- the change of free device
    memory around warmed-up forward, no-allocation forward, backward and stack calls (0 bytes:
    every buffer is the caller's); (2) the caller's buffers per item -- Q, K, V, O and the
    workspace linformer_workspace_size asks for, per item at the largest batch one call takes,
    plus E once; (3) standard attention written with torch operations (n x n fp32 scores and
    bf16 probabilities), its peak beyond Q, K, V, O from torch's allocator at batch 1 and 2
    (the difference is the per-item bytes), where one item fits on the device; where it does not
    (n = 65536), the same recipe's size as a model (6 n^2 bytes per head), labelled as such.
    The in-repo dense comparator streams the keys and keeps no n x n matrix: its footprint is
    Q, K, V, O, and it allocates nothing either (measured like (1))."""
    H, d = 12, 64
    free, total = torch.cuda.mem_get_info()
    budget = free - (1 << 30)   # leave 1 GiB for the runtime
    bf = torch.bfloat16

    # (1) the library's own device allocations, after warm-up
    B, n, k = 4, 4096, 256
    p = L.problem(B, H, n, d, k, synth.DT_BF16, synth.SHARE_LAYERWISE, 0.0)
    Q = torch.randn(B, H, n, d, device="cuda").to(bf)
    K = torch.randn(B, H, n, d, device="cuda").to(bf)
    V = torch.randn(B, H, n, d, device="cuda").to(bf)
    E = (torch.randn(1, k, n, device="cuda") / 16).to(bf)
    O = torch.empty_like(Q)
    wsb = L.linformer_workspace_size(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    f32 = lambda *shape: torch.empty(*shape, dtype=torch.float32, device="cuda")
    dQ, dK, dV, dE = f32(B, H, n, d), f32(B, H, n, d), f32(B, H, n, d), f32(1, k, n)
    bwb = L.linformer_backward_workspace_size(p)
    bws = torch.empty(bwb, dtype=torch.uint8, device="cuda")
    st = L.stack(2, 1024, 768, 12, 256, 2, False, 0.0)
    X = torch.randn(2, 1024, 768, device="cuda").to(bf)
    Wq = (torch.randn(2, 3 * 768, 768, device="cuda") * 0.02).to(bf)
    Wo = (torch.randn(2, 768, 768, device="cuda") * 0.02).to(bf)
    Es = (torch.randn(1, 256, 1024, device="cuda") / 16).to(bf)
    Y = torch.empty(2, 1024, 768, dtype=bf, device="cuda")
    swb = L.linformer_stack_workspace_size(st)
    sws = torch.empty(swb, dtype=torch.uint8, device="cuda")
    lib_alloc = {
        "forward": library_allocation(torch, lambda: L.linformer_forward(p, Q, K, V, E, None, None, O, ws, wsb)),
        "forward_noalloc": library_allocation(torch, lambda: L.linformer_forward_noalloc(p, Q, K, V, E, None, None, O)),
        "backward": library_allocation(torch, lambda: L.linformer_backward(p, Q, K, V, E, None, None, O, dQ, dK, dV, dE, None, bws, bwb)),
        "stack": library_allocation(torch, lambda: L.linformer_stack_forward(st, X, Wq, Wo, Es, None, Y, sws, swb)),
        "dense_comparator": library_allocation(torch, lambda: L.attention_dense_forward(p, Q, K, V, None, O)),
    }
    log(f"device memory the library allocates per call after warm-up: {lib_alloc}")
    del Q, K, V, E, O, ws, dQ, dK, dV, dE, bws, X, Wq, Wo, Es, Y, sws
    torch.cuda.empty_cache()

    rows = []
    for n in (512, 4096, 65536):
        for k in (128, 256):
            # (2) the caller's buffers, per item at the largest batch one call takes (the
            # position split, and with it the partial sums, shrinks as the batch grows)
            bmax = min(4096, ((1 << 31) - 1) // (H * n * d))
            pb = L.problem(bmax, H, n, d, k, synth.DT_BF16, synth.SHARE_LAYERWISE, 0.0)
            qkvo = 4 * H * n * d * 2
            lin_item = qkvo + L.linformer_workspace_size(pb) / bmax
            lin_fixed = k * n * 2
            # (3) standard attention: measured where one item fits, else the recipe's size
            if n <= 4096:
                # the first batched product allocates the BLAS workspace once: not per item
                standard_attention_bytes(torch, 1, H, n, d)
                s1 = standard_attention_bytes(torch, 1, H, n, d)
                s2 = standard_attention_bytes(torch, 2, H, n, d)
                std_extra, std_kind = s2 - s1, "measured: torch operations, peak over Q, K, V, O, slope over batch 1 -> 2"
            else:
                std_extra, std_kind = 6 * H * n * n, "model: 6 n^2 bytes per head (fp32 scores + bf16 probabilities); one item does not fit"
            std_item = qkvo + std_extra
            row = {"n": n, "k": k, "linformer_bytes_per_item": int(lin_item),
                   "standard_bytes_per_item": int(std_item), "standard_kind": std_kind,
                   "streamed_dense_bytes_per_item": qkvo,
                   "linformer_max_batch": int((budget - lin_fixed) // lin_item),
                   "standard_max_batch": int(budget // std_item),
                   "streamed_dense_max_batch": int(budget // qkvo),
                   "bytes_per_item_ratio_vs_standard": round(std_item / lin_item, 2),
                   "max_batch_per_call": bmax}
            row["max_batch_ratio_vs_standard"] = (
                round(row["linformer_max_batch"] / row["standard_max_batch"], 2)
                if row["standard_max_batch"] > 0 else None)
            rows.append(row)
            log(f"n={n:6d} k={k}: Linformer {lin_item / 2**20:9.2f} MiB/item "
                f"(max batch {row['linformer_max_batch']}), standard {std_item / 2**20:10.2f} MiB/item "
                f"(max batch {row['standard_max_batch']}; {std_kind.split(':')[0]}), ratio "
                f"{row['max_batch_ratio_vs_standard']}")
    print(json.dumps({"memory": rows, "library_allocation_bytes": lib_alloc,
                      "free_bytes": free, "total_bytes": total, "budget_bytes": budget,
                      "config": {"heads": H, "head_dim": d, "share": "layerwise",
                                 "dtype": "bf16"},
                      "source_sha": source_hashes(),
                      "command": "python bench.py " + " ".join(sys.argv[1:])}), flush=True)


PEAK_F32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix-core peak (published)


def run_backward(args, L, synth, torch, np):
    """linformer_backward on a workload's inputs with a random upstream gradient: gradients of Q,
    K, V, E, F (fp32 accumulation; every product on the bf16 matrix cores as split pairs).
    Algorithmic work per (b, h): 22 n k d flops, eleven products of 2 n k d (Kbar, Vbar
    recomputed; scores, dP, dQ; dVbar, dKbar; dE, dF; dK, dV).  Executed matrix-core work: the
    slot-block kernel computes the scores and dP a second time (so no n x k matrix is stored),
    thirteen products in all, and a product takes 1 + (one per fp32 operand) bf16 products
    (hi.hi, lo.hi, hi.lo), the roofline's basis against the bf16 peak."""
    wl = synth.WORKLOADS[args.workload]
    inp = synth.make_inputs(wl)
    td = torch.bfloat16 if wl.dtype == synth.DT_BF16 else torch.float32
    dev = lambda x: torch.from_numpy(x).to(td).cuda()
    p = L.problem(wl.batch, wl.heads, wl.n, wl.d, wl.k, wl.dtype, wl.share, 0.0)
    Q, K, V, E = dev(inp.Q), dev(inp.K), dev(inp.V), dev(inp.E)
    F = dev(inp.F) if inp.F is not None else None
    lens = (torch.tensor(inp.lengths, dtype=torch.int32, device="cuda")
            if inp.lengths is not None else None)
    dO = dev(np.random.default_rng(1).standard_normal((wl.batch, wl.heads, wl.n, wl.d)).astype(np.float32))
    f32 = lambda shape: torch.empty(shape, dtype=torch.float32, device="cuda")
    shp = (wl.batch, wl.heads, wl.n, wl.d)
    dQ, dK, dV, dE = f32(shp), f32(shp), f32(shp), f32(tuple(inp.E.shape))
    dF = f32(tuple(inp.F.shape)) if inp.F is not None else None
    wsb = L.linformer_backward_workspace_size(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        L.linformer_backward(p, Q, K, V, E, F, lens, dO, dQ, dK, dV, dE, dF, ws, wsb,
                             stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    flops = 22.0 * wl.batch * wl.heads * wl.n * wl.k * wl.d
    tf = flops / (ms * 1e-3) / 1e12
    # operands of the thirteen executed products, True where fp32 (inputs in x, the computed
    # intermediates Kbar, Vbar, P, dS, dKbar, dVbar in fp32): Kbar = E K, Vbar = F V,
    # S = Q Kbar^T, dP = dO Vbar^T, dQ = dS Kbar (query-block kernel), S and dP again,
    # dVbar = P^T dO, dKbar = dS^T Q (slot-block kernel), dE = dKbar K^T, dF = dVbar V^T,
    # dK = E^T dKbar, dV = F^T dVbar
    x = wl.dtype != synth.DT_BF16
    ops = [(x, x), (x, x), (x, True), (x, True), (True, True), (x, True), (x, True),
           (True, x), (True, x), (True, x), (True, x), (x, True), (x, True)]
    mult = sum(1 + int(a) + int(b) for a, b in ops)
    executed = 2.0 * mult * wl.batch * wl.heads * wl.n * wl.k * wl.d
    etf = executed / (ms * 1e-3) / 1e12
    tokens = wl.batch * wl.n
    log(f"backward: {ms * 1e3:.1f} us/step ({tokens / (ms / 1e3):.3e} tokens/s), {tf:.1f} TFLOP/s "
        f"fp32-equivalent, {etf:.1f} TFLOP/s executed bf16")
    print(json.dumps({
        "metric": "Linformer backward (dQ, dK, dV, dE, dF) tokens/s", "value": round(tokens / (ms / 1e3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "inputs": "bf16" if wl.dtype == synth.DT_BF16 else "f32"},
        "roofline": {"bound": "mfma", "achieved": round(etf, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(etf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "whole backward step", "executed_bf16_flops": executed,
                     "algorithmic_flops": flops, "fp32_equivalent_tflops": round(tf, 1),
                     "fp32_equivalent_frac_of_f32_peak": round(tf / PEAK_F32_MFMA_TFLOPS, 4),
                     "basis": "executed: each product as 1 + (fp32 operands) bf16 products"},
        "time_basis": "HIP events around the timed back-to-back backward calls",
        "source_sha": source_hashes(),
        "command": "python bench.py " + " ".join(sys.argv[1:]),
        "device": torch.cuda.get_device_name(0)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--replicas", type=int, default=0,
                    help="input replicas rotated over the steps; 0 = enough for >= 1 GiB of "
                         "inputs, so the 256 MB last-level cache cannot serve them")
    ap.add_argument("--workload", default="long_b8_h12_n4096_k256_unshared_padded")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--kernel-iters", type=int, default=20)
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the bench line: forward time over n for B1 H12 and "
                         "k = 128, 256 (layerwise E = F), with the dense comparator up to n = 16384")
    ap.add_argument("--proj", choices=("dense", "conv"), default="dense",
                    help="sequence compression: the dense projection E, F (default) or the "
                         "window-s stride-s convolution (no E read)")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the bench line: time the backward pass on the workload")
    ap.add_argument("--memory", action="store_true",
                    help="instead of the bench line: device memory per batch item and the largest "
                         "batch that fits, Linformer against standard attention")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run a plain device copy of this many MB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: --gpus N > 1 is not supported (every kernel runs on "
              "one device's share of the work)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from efficient_transformer_attention_seq_amd import linformer as L
    from efficient_transformer_attention_seq_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    L.lib()  # fail loudly if the HIP library is missing
    if args.copy_mb:
        src = torch.empty(args.copy_mb * 1 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_mb} MiB x3")
        return
    if args.sweep:
        run_sweep(L, synth, torch, np)
        return
    if args.memory:
        run_memory(L, synth, torch, np)
        return
    if args.backward:
        run_backward(args, L, synth, torch, np)
        return
    if args.workload in synth.STACK_WORKLOADS:
        run_stack_bench(args, L, synth, torch, np)
        return
    wl = synth.WORKLOADS[args.workload]
    log(f"workload {wl}")
    t0 = time.time()
    inp = synth.make_inputs(wl)
    log(f"inputs drawn in {time.time() - t0:.1f}s; lengths={None if inp.lengths is None else inp.lengths.tolist()}")

    td = torch.bfloat16 if wl.dtype == synth.DT_BF16 else torch.float32

    def dev(x):
        return torch.from_numpy(x).to(td).cuda()

    p = L.problem(wl.batch, wl.heads, wl.n, wl.d, wl.k, wl.dtype, wl.share, 0.0)
    if args.replicas <= 0:
        esz = 2 if wl.dtype == synth.DT_BF16 else 4
        per = (3 * wl.batch * wl.heads * wl.n * wl.d +
               wl.e_heads * wl.k * wl.n * (2 if wl.separate_f else 1)) * esz
        args.replicas = max(2, -(-(1 << 30) // per))
    log(f"{args.replicas} input replicas")
    reps = []
    for r in range(args.replicas):
        reps.append(dict(Q=dev(inp.Q), K=dev(inp.K), V=dev(inp.V), E=dev(inp.E),
                         F=dev(inp.F) if inp.F is not None else None))
    lens = (torch.tensor(inp.lengths, dtype=torch.int32, device="cuda")
            if inp.lengths is not None else None)
    conv = args.proj == "conv"
    if conv:   # window weights replace E and F (per head, as E and F are for this workload)
        s_win = wl.n // wl.k
        wE = synth.conv_weights(wl.e_heads, s_win, seed=11)
        wF = synth.conv_weights(wl.e_heads, s_win, seed=12) if wl.separate_f else None
        for r in reps:
            r["E"] = dev(wE)
            r["F"] = dev(wF) if wF is not None else None
    O = torch.empty(wl.batch, wl.heads, wl.n, wl.d, dtype=td, device="cuda")
    wsb = L.linformer_workspace_size(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    kb, vb = L.linformer_kv_sizes(p)
    Kbar = torch.empty(kb, dtype=torch.uint8, device="cuda")
    Vbar = torch.empty(vb, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        r = reps[i % len(reps)]
        if conv:
            L.linformer_forward_conv(p, r["Q"], r["K"], r["V"], r["E"], r["F"], lens, O, ws, wsb,
                                     stream=stream)
        else:
            L.linformer_forward(p, r["Q"], r["K"], r["V"], r["E"], r["F"], lens, O, ws, wsb,
                                stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = ev0.elapsed_time(ev1) / args.steps
    tokens = wl.batch * wl.n
    log(f"forward: {ms * 1e3:.1f} us/step ({tokens / (ms / 1e3):.3e} tokens/s), wall {wall:.3f}s")

    # ---- per-kernel timing of the two halves, on the same stream, with rotated replicas
    def time_half(kind, iters):
        for i in range(3):
            run_half(kind, i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(iters):
            run_half(kind, i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters * 1e3  # us

    def run_half(kind, i):
        r = reps[i % len(reps)]
        if kind == "project" and conv:
            L.linformer_project_kv_conv(p, r["K"], r["V"], r["E"], r["F"], lens, Kbar, Vbar,
                                        stream=stream)
        elif kind == "project":
            L.linformer_project_kv(p, r["K"], r["V"], r["E"], r["F"], lens, Kbar, Vbar, ws,
                                   wsb, stream=stream)
        else:
            L.linformer_attend(p, r["Q"], Kbar, Vbar, lens, O, stream=stream)

    fused = uses_fused(wl, conv)
    kern = {}
    if fused:
        # one launch per step: the fused kernel is the step
        byts, flops = step_algorithmic(wl, conv)
        us = ms * 1e3
        kern["fused"] = dict(us=us, bytes=byts, flops=flops, gbs=byts / (us * 1e-6) / 1e9,
                             tflops=flops / (us * 1e-6) / 1e12)
        dom, dom_name = "fused", "fused_bf16_kernel"
    else:
        run_half("project", 0)
        for kind in ("project", "attend"):
            us = time_half(kind, args.kernel_iters)
            byts, flops = algorithmic(wl, kind, conv)
            kern[kind] = dict(us=us, bytes=byts, flops=flops, gbs=byts / (us * 1e-6) / 1e9,
                              tflops=flops / (us * 1e-6) / 1e12)
        # roofline of the dominant single kernel: the attention kernel (one launch per half; the
        # projection half is one kernel, plus the split fixup for three or more splits)
        if wl.dtype == 1:
            dom, dom_name = "attend", "attend_bf16_kernel"
        else:
            dom, dom_name = "attend_f32", "attend_f32_kernel"
    for kind, kv in kern.items():
        log(f"{kind}: {kv['us']:.1f} us/launch, {kv['gbs']:.0f} GB/s algorithmic, "
            f"{kv['tflops']:.1f} TFLOP/s")
    kd = kern["attend" if dom == "attend_f32" else dom]
    traffic = traffic_bytes(dom, wl.name)
    rp_us = rocprof_us(dom, wl.name)
    roofline = {"bound": "hbm", "achieved": round(kd["gbs"], 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(kd["gbs"] / PEAK_HBM_GBS, 4),
                "traffic": traffic, "kernel": dom_name, "avg_us": round(kd["us"], 2),
                "algorithmic_bytes": kd["bytes"],
                # matrix-core rate (bf16 kernels), or the fp32 vector rate (fp32 kernels)
                "mfma_tflops": round(kd["tflops"], 1) if wl.dtype == 1 else None,
                "mfma_frac": round(kd["tflops"] / PEAK_BF16_TFLOPS, 4) if wl.dtype == 1 else None,
                "vector_f32_frac": None if wl.dtype == 1 else
                round(kd["tflops"] / PEAK_F32_TFLOPS, 4),
                # the same bytes over the committed profiler duration of this kernel source
                "rocprof_us": None if rp_us is None else round(rp_us, 2),
                "frac_rocprof": None if rp_us is None else
                round(kd["bytes"] / (rp_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    step_bytes, step_flops = step_algorithmic(wl, conv)
    peak_flops = (PEAK_BF16_TFLOPS if wl.dtype == 1 else PEAK_F32_TFLOPS) * 1e12
    roof_us = max(step_bytes / (PEAK_HBM_GBS * 1e9), step_flops / peak_flops) * 1e6

    # the same roofline over the valid work only (rows past each length do no work: the
    # projection skips them and the attention only zero-fills them)
    valid = None
    if inp.lengths is not None:
        Ls = [int(x) for x in inp.lengths]
        n_mats = wl.e_heads * (2 if wl.separate_f else 1)
        eb = 2 if wl.dtype == synth.DT_BF16 else 4
        vtok = sum(Ls)
        vbytes = 4 * wl.heads * wl.d * eb * vtok + (0 if conv else n_mats * wl.k * wl.n * eb)
        vflops = 8.0 * wl.heads * wl.k * wl.d * vtok
        vroof = max(vbytes / (PEAK_HBM_GBS * 1e9), vflops / peak_flops) * 1e6
        valid = {"tokens": vtok, "tokens_per_s": round(vtok / (ms / 1e3), 1),
                 "algorithmic_bytes": vbytes, "flops": vflops, "roofline_us": round(vroof, 2),
                 "frac": round(vroof / (ms * 1e3), 4)}
        log(f"valid work: {vtok} tokens, roofline {vroof:.1f} us, frac {vroof / (ms * 1e3):.3f}")

    copy_gbs = copy_ceiling(torch)
    log(f"device copy: {copy_gbs:.0f} GB/s (read + write)")

    dense = None
    if not args.no_dense and not conv and wl.dtype == synth.DT_BF16 and wl.n <= 16384:
        Od = torch.empty_like(O)
        for i in range(2):
            L.attention_dense_forward(p, reps[i % len(reps)]["Q"], reps[i % len(reps)]["K"],
                                      reps[i % len(reps)]["V"], lens, Od, stream=stream)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nd = max(3, args.steps // 4)
        a.record(stream)
        for i in range(nd):
            r = reps[i % len(reps)]
            L.attention_dense_forward(p, r["Q"], r["K"], r["V"], lens, Od, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        dms = a.elapsed_time(b) / nd
        dense = {"ms": round(dms, 4), "speedup_vs_dense": round(dms / ms, 2)}
        log(f"dense O(n^2) attention: {dms * 1e3:.1f} us/step, Linformer speedup {dms / ms:.2f}x")

    cpu = None
    if not args.no_cpu_baseline and not conv:
        log("timing the float64 oracle on the host cores ...")
        cpu = cpu_baseline(inp)
        log(f"oracle: {cpu['value']:.3e} tokens/s on {cpu['cores']} threads ({cpu['sample']})")

    out = {
        "metric": METRIC,
        "value": round(tokens / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == synth.DT_BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "heads": wl.heads, "seq_len": wl.n,
                   "head_dim": wl.d, "k": wl.k, "share": synth.SHARE_NAMES[wl.share],
                   "padded": wl.padded, "replicas": args.replicas,
                   "compression": "conv (window n/k, per-head weights)" if conv else "dense E, F"},
        "roofline": roofline,
        "step_roofline": {"algorithmic_bytes": step_bytes, "roofline_us": round(roof_us, 2),
                          "frac": round(roof_us / (ms * 1e3), 4)},
        "valid_work_roofline": valid,
        "kernels_us": {k: round(v["us"], 2) for k, v in kern.items()},
        "bytes_basis": "step_roofline: the scope table's count -- Q, K, V, O over the padded "
                       "length n and each distinct E/F matrix once (Kbar/Vbar excluded); "
                       "valid_work_roofline: the same over the valid rows only; roofline (one "
                       "kernel): its own inputs and outputs over the padded length, Kbar and Vbar "
                       "(bf16) included for the two-launch halves",
        "time_basis": "ms_per_step: HIP events around the timed back-to-back forward calls on "
                      "the launch stream; kernels_us / roofline.avg_us: HIP events around "
                      "back-to-back launches of one half, or the step itself when one fused "
                      "kernel is the step (includes the dispatch gap between launches); "
                      "roofline.rocprof_us: average kernel duration in the committed rocprofv3 "
                      "trace at this kernel source (profiles/kernel_times.txt)",
        "source_sha": source_hashes(),
        "command": "python bench.py " + " ".join(sys.argv[1:]),
        "dense_comparator": dense,
        "copy_ceiling_gbs": round(copy_gbs, 1),
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(0),
        "wall_s": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
