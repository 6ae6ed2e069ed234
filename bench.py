#!/usr/bin/env python3
"""Throughput of the chunked gated delta-rule forward on one MI355X.

A step is one full forward (intra-chunk kernel, chunk-to-chunk chain, output kernel) over
one batch of seeded synthetic inputs of the KDA workload B=1, T=8192, H=16, K=V=128,
chunk 128, with a std-0.1 initial state and the final state returned.  Inputs are
resident in HBM before timing starts; three input sets are rotated so that a step does
not find its inputs in the 256 MB memory-attached cache from the previous step.

Prints one JSON line: tokens/s for the whole job, ms per step, per-kernel durations from
HIP events on the launch stream, the roofline of the dominant kernel, and the fp64
oracle timed on the host cores as a CPU baseline.

    python bench.py [--steps K] [--warmup W] [--workload kda_t8192] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "forward tokens/s + % bf16 MFMA peak, KDA T=8192 H=16 K=V=128"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
SEED_BASE = 1003            # workload seeds: 1000 + position of the workload in the list


def nominal_flops(w, lengths):
    """The headline work F_nom of the method as the page writes it, per chunk of n tokens and
    head (K = V = 128): A, A2 and w as full n x n products (n^2 K each), u and A2 v_new
    (n^2 V each), w S, qg S and kg^T v_new (n K V each), two flops per multiply-add, plus
    n^3 / 3 for the inverse.  Tail chunks count with their real n."""
    K, V, C, H = w.K, w.V, w.chunk_size, w.H
    f = 0.0
    for L in lengths:
        for c0 in range(0, L, C):
            n = min(C, L - c0)
            f += H * (2.0 * (3 * n * n * K + 2 * n * n * V + 3 * n * K * V) + n ** 3 / 3.0)
    return f


def min_flops(w, lengths):
    """F_min: F_nom with the triangular products counted once per pair (A, A2, w, u and A2 v_new
    are lower-triangular n x n products, so their n^2 terms halve)."""
    K, V, C, H = w.K, w.V, w.chunk_size, w.H
    f = 0.0
    for L in lengths:
        for c0 in range(0, L, C):
            n = min(C, L - c0)
            f += H * (2.0 * (1.5 * n * n * K + n * n * V + 3 * n * K * V) + n ** 3 / 3.0)
    return f


def compulsory_bytes(w, lengths):
    """The forward's compulsory HBM bytes: q, k, v and o in bf16, g in fp32 (per dimension or one
    per token and head), beta in fp32, the initial state when given and the final state, fp32."""
    tokens = sum(lengths)
    gate_bytes = 4 * w.K if w.per_dim_gate else 4
    state = w.K * w.V * 4
    return (tokens * w.H * (2 * 2 * w.K + 2 * 2 * w.V + gate_bytes + 4)
            + len(lengths) * w.H * state * (2 if w.initial_state else 1))


def kernel_work(w, lengths):
    """Algorithmic flops and compulsory bytes per kernel of this implementation, in which the
    chunk step is re-associated (S' = exp(gamma_C) S - P S + B, o = Q S + U).  Per chunk of n
    tokens and head:
      intra   A, A2 (full n x n products, 2 n^2 K each), the inverse (n^3 / 3), w (2 n^2 K),
              u (2 n^2 V), P = kg^T w (2 n K^2), B = kg^T u (2 n K V), A2 w (2 n^2 K),
              A2 u (2 n^2 V)
      chain   P S (2 K^2 V, whatever n)
      output  Q S (2 n K V)
    Bytes are the compulsory ones each kernel owns: q, k, v, g, beta read by the intra
    kernel, the initial and final state moved by the chain, o written by the output kernel;
    intermediates are not counted."""
    K, V, C, H = w.K, w.V, w.chunk_size, w.H
    f = {"intra": 0.0, "chain": 0.0, "output": 0.0}
    for L in lengths:
        for c0 in range(0, L, C):
            n = min(C, L - c0)
            f["intra"] += H * (2.0 * (2 * n * n * K) + n ** 3 / 3.0 + 2.0 * (n * n * K + n * n * V)
                               + 2.0 * (n * K * K + n * K * V) + 2.0 * (n * n * K + n * n * V))
            f["chain"] += H * 2.0 * K * K * V
            f["output"] += H * 2.0 * n * K * V
    tokens = sum(lengths)
    gate_bytes = 4 * K if w.per_dim_gate else 4
    b = {"intra": tokens * H * (2 * 2 * K + 2 * V + gate_bytes + 4),
         "chain": len(lengths) * H * K * V * 4 * (2 if w.initial_state else 1),
         "output": tokens * H * 2 * V}
    return f, b


KERNEL_SOURCES = {"intra": ("cdr_intra.hip", "cdr_common.h"),
                  "prep": ("cdr_bwd.hip", "cdr_common.h"),
                  "chains": ("cdr_bwd.hip", "cdr_common.h"),
                  "local": ("cdr_bwd.hip", "cdr_common.h"),
                  "chain": ("cdr_chain.hip", "cdr_common.h"),
                  "output": ("cdr_chain.hip", "cdr_common.h"),
                  "decode": ("cdr_decode.hip", "cdr_common.h")}


def source_hash(kernel):
    """Hash of the sources a kernel is built from (counter summaries are tied to it)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "chunked_gated_delta_chunk_amd", "csrc", name), "rb") as fh:
            h.update(name.encode() + fh.read())
    return h.hexdigest()[:16]


def load_counters(kernel, workload, what="hbm_traffic", field="hbm_bytes"):
    """A per-launch figure from a committed counter summary (profiles/<workload>_<what>.json),
    if the summary was taken on the current sources of the kernel."""
    path = os.path.join(ROOT, "profiles", f"{workload}_{what}.json")
    try:
        with open(path) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    rec = data.get(workload, {}).get(kernel)
    if not rec or rec.get("source_sha") != source_hash(kernel):
        return None
    return rec.get(field)


def load_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it matches the sources."""
    return load_counters(kernel, workload)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def decode_bytes(w):
    """Compulsory HBM bytes of one decode call: every state read once and written once per
    stored position (64 KiB each at K = V = 128), the token inputs (q, k per key head; v, g,
    beta per value head), o, and the slot indices."""
    state = w.V * w.K * 4
    writes = 1 if w.index_cols == 0 else min(w.T, w.index_cols)
    per_tok = (w.H * w.K * 2 * 2
               + w.HV * (w.V * 2 + (w.K * 4 if w.per_dim_gate else 4) + 4 + w.V * 2))
    idx = w.N * max(w.index_cols, 1) * 4 + (w.N * 4 if w.index_cols else 0)
    return w.N * w.HV * state * (1 + writes) + w.tokens * per_tok + idx


def bench_decode(name, steps, warmup):
    """Time one decode workload: a call is one kernel over the batch, the pool updated in
    place.  Slot sets are rotated (disjoint, up to 4) so that a call does not find the
    states of the previous call in cache."""
    import torch
    import chunked_gated_delta_chunk_amd as cdr
    from chunked_gated_delta_chunk_amd.synth import DECODE_WORKLOADS, decode_workload_inputs
    w = DECODE_WORKLOADS[name]
    dev = torch.device("cuda:0")
    host = decode_workload_inputs(w, seed=2000 + list(DECODE_WORKLOADS).index(name))
    d = host.to(dev)
    per = w.N * max(w.index_cols, 1)
    nsets = max(1, min(4, w.num_slots // per))
    perm = torch.randperm(w.num_slots, generator=torch.Generator().manual_seed(7)).to(torch.int32)
    calls = []
    for i in range(nsets):
        idx = perm[i * per:(i + 1) * per].reshape(d.ssm_state_indices.shape).contiguous().to(dev)
        calls.append(cdr.PreparedRecurrent(d.q, d.k, d.v, d.g, d.beta, cu_seqlens=d.cu_seqlens,
                                           use_qk_l2norm_in_kernel=w.qk_l2norm,
                                           state_pool=d.state_pool, ssm_state_indices=idx,
                                           num_accepted_tokens=d.num_accepted_tokens))
    for i in range(warmup):
        calls[i % nsets]()
    torch.cuda.synchronize()
    # a spin kernel queued first keeps the GPU busy while the host queues the calls, so the
    # timed launches run back to back; the events bracket the K launches and nothing else
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(steps * 200e-6 * 2.1e9))
    start.record()
    for i in range(steps):
        calls[i % nsets]()
    end.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(end) / steps * 1e3
    nbytes = decode_bytes(w)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": name, "us_per_call": round(us, 2),
            "tokens_per_s": round(w.tokens / (us * 1e-6), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": load_traffic("decode", name), "kernel": "decode_kernel",
                         "algorithmic_bytes": nbytes},
            "config": {"N": w.N, "T": w.T, "H": w.H, "HV": w.HV, "K": w.K, "V": w.V,
                       "num_slots": w.num_slots, "index_cols": w.index_cols,
                       "qk_l2norm": w.qk_l2norm, "slot_sets_rotated": nsets}}


def backward_work(w, lengths):
    """Per-stage flops of the backward (products counted once, as full products like the
    forward's nominal count) and its compulsory bytes; n = rows of each chunk."""
    K, V = w.K, w.V
    fl = {"prep": 0.0, "chains": 0.0, "local": 0.0}
    for L in lengths:
        nchunks = (L + w.chunk_size - 1) // w.chunk_size
        for c in range(nchunks):
            n = min(w.chunk_size, L - c * w.chunk_size)
            fl["prep"] += 2 * (2 * n * n * K + n ** 3 / 3 + n * n * K + n * n * V + n * K * K + n * K * V
                               + n * n * V + 2 * n * K * V)
            fl["chains"] += 2 * 2 * K * K * V
            fl["local"] += 2 * (n * K * V + n * n * V + n * K * V + n * n * V + 3 * n * K * V + n * n * V
                                + n * n * K + n * n * V + n * n * K + 2 * n ** 3 + 4 * n * n * K)
    fl = {k: v * w.H for k, v in fl.items()}
    per_tok = 4 * 2 * K + (4 * K if w.per_dim_gate else 4) + 4 + 4 * 4 * K + (4 * K if w.per_dim_gate else 4) + 4
    nbytes = w.tokens * w.H * per_tok + (2 * len(lengths) * w.H * K * V * 4 if w.initial_state else 0)
    return fl, nbytes


def bench_backward(name, steps, warmup):
    """Time the backward of one forward workload: one call is the three stages (prep, the two
    state chains, local gradients), events between the stages on the launch stream."""
    import torch
    import chunked_gated_delta_chunk_amd as cdr
    from chunked_gated_delta_chunk_amd.synth import WORKLOADS, workload_inputs
    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    host = workload_inputs(w, seed=1000 + list(WORKLOADS).index(name) + 1)
    gen = torch.Generator("cpu").manual_seed(7)
    do = torch.randn(tuple(host.v.shape), generator=gen).to(torch.bfloat16)
    N = w.N
    dht = 0.1 * torch.randn(N, w.H, w.V, w.K, generator=gen)
    d = host.to(dev)
    call = cdr.PreparedBackward(d.q, d.k, d.v, d.g, d.beta, do.to(dev), dht=dht.to(dev),
                                initial_state=d.initial_state, cu_seqlens=d.cu_seqlens,
                                chunk_size=w.chunk_size)
    stages = (cdr.BWD_PREP, cdr.BWD_CHAINS, cdr.BWD_LOCAL)
    names = ("prep", "chains", "local")
    for _ in range(warmup):
        for st in stages:
            call(st)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record()
        for j, st in enumerate(stages):
            call(st)
            ev[i][j + 1].record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    kus = {nm: sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)) / steps * 1e3
           for j, nm in enumerate(names)}
    lengths = list(w.lengths) if w.lengths is not None else [w.T] * w.B
    fl, nbytes = backward_work(w, lengths)
    dom = max(names, key=lambda n: kus[n])
    tf = fl[dom] / (kus[dom] * 1e-6) / 1e12
    return {"workload": name, "ms_per_call": round(ms, 4), "tokens_per_s": round(w.tokens / (ms * 1e-3), 1),
            "per_kernel_us": {k: round(v, 2) for k, v in kus.items()},
            "gflop": {k: round(v / 1e9, 2) for k, v in fl.items()},
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": load_traffic(dom, name + "_backward"),
                         "kernel": "bwd_" + dom, "duration_us": round(kus[dom], 2)},
            "compulsory_bytes": nbytes}


def bench_context_parallel(name, ranks, steps, warmup):
    """One rank's share of the workload when its sequence is split over `ranks` ranks: the
    segment summary (M, X) of T / ranks tokens, and the merge of `ranks` summaries."""
    import torch
    import chunked_gated_delta_chunk_amd as cdr
    from chunked_gated_delta_chunk_amd.synth import WORKLOADS, make_inputs
    w = WORKLOADS[name]
    seg = w.T // ranks
    inp = make_inputs(1, seg, w.H, w.K, w.V, seed=77, chunk_size=w.chunk_size).to("cuda:0")
    p = cdr.make_problem(1, seg, w.H, w.K, w.V, 1, True, w.chunk_size, w.K ** -0.5, False, True, False)
    ws = torch.empty(cdr.workspace_bytes(p), dtype=torch.uint8, device="cuda:0")
    for _ in range(warmup):
        M, X = cdr.segment_map(inp.q, inp.k, inp.v, inp.g, inp.beta, chunk_size=w.chunk_size, workspace=ws)
    Ms, Xs = M.expand(ranks, -1, -1, -1).contiguous(), X.expand(ranks, -1, -1, -1).contiguous()
    for _ in range(warmup):
        cdr.merge_states(Ms, Xs)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record()
    for _ in range(steps):
        cdr.segment_map(inp.q, inp.k, inp.v, inp.g, inp.beta, chunk_size=w.chunk_size, workspace=ws)
    e[1].record()
    for _ in range(steps):
        cdr.merge_states(Ms, Xs)
    e[2].record()
    torch.cuda.synchronize()
    return {"workload": f"{name}, one of {ranks} ranks ({seg} tokens x {w.H} heads)",
            "segment_map_us": round(e[0].elapsed_time(e[1]) / steps * 1e3, 2),
            "merge_us": round(e[1].elapsed_time(e[2]) / steps * 1e3, 2),
            "summary_bytes_per_rank": w.H * (w.K * w.K + w.V * w.K) * 4}


def cpu_baseline(inp, w, budget_s):
    """Time the fp64 oracle on the host: all heads, a prefix of the tokens sized to the
    time budget (all tokens when it fits)."""
    import numpy as np  # noqa: F401
    import oracle
    threads = oracle.num_threads()
    chains = w.N * w.H
    T = w.tokens

    def run(tsub):
        sl = lambda t: None if t is None else t[:, :tsub].contiguous()  # noqa: E731
        # packed sequences: the prefix ends every sequence at token tsub (later ones empty)
        cu = None if inp.cu_seqlens is None else inp.cu_seqlens.clamp(max=tsub)
        t0 = time.perf_counter()
        oracle.recurrent_fwd(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.g), sl(inp.beta),
                             initial_state=inp.initial_state, cu_seqlens=cu)
        return time.perf_counter() - t0

    probe = min(T, 512)
    dt = run(probe)
    tsub = T if dt * T / probe <= budget_s else max(probe, int(budget_s / dt * probe) // 64 * 64)
    if tsub != probe:
        dt = run(tsub)
    # repeat a short sample until about a second of wall time has been measured
    reps = max(1, min(20, int(1.0 / max(dt, 1e-3))))
    if reps > 1:
        dt = min(dt, min(run(tsub) for _ in range(reps - 1)))
    return {"value": tsub * w.B / dt if w.lengths is None else tsub / dt, "unit": "tokens/s",
            "cores": min(threads, chains), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": (f"fp64 per-token recurrence (C, OpenMP over {chains} (sequence, head) chains) "
                       f"on the first {tsub} of {T} tokens of every head, best of {reps} runs, "
                       f"{dt:.3f} s wall each")}


EV_STRIDE = 10        # timed steps per step with per-kernel events
CLOCK_WARMUP_S = 0.3  # untimed forward calls before the warmup steps (clock ramp)
COLD_STEPS = 20       # event-timed single forwards, flushed and warm
GRAPH_REPLAYS = 200   # replays of one captured forward (same input set)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="kda_t8192")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=8.0, help="seconds of oracle wall time")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode workloads")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the backward of the workload and print its JSON line")
    ap.add_argument("--decode-only", default=None, metavar="NAME",
                    help="time only this decode workload and print its JSON line")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (reference for the "
                         "HBM byte counters) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy * 2 ** 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n, "calibrate_copy_bytes_written": n, "launches": 3}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path; the forward "
              "would shard over heads and sequences with no exchange between them",
              file=sys.stderr)
        sys.exit(2)

    if args.backward_only:
        r = bench_backward(args.workload, args.steps, args.warmup)
        r.update({"metric": "backward tokens/s", "unit": "tokens/s", "value": r["tokens_per_s"],
                  "higher_is_better": True, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                  "dtype": "bf16", "data": "synthetic"})
        print(json.dumps(r), flush=True)
        return
    if args.decode_only:
        r = bench_decode(args.decode_only, args.steps, args.warmup)
        r.update({"metric": "decode tokens/s + % HBM peak", "unit": "tokens/s",
                  "value": r["tokens_per_s"], "higher_is_better": True, "n_gpus": 1,
                  "steps": args.steps, "warmup": args.warmup, "dtype": "f32",
                  "data": "synthetic"})
        print(json.dumps(r), flush=True)
        return

    import torch
    import chunked_gated_delta_chunk_amd as cdr
    from chunked_gated_delta_chunk_amd.synth import WORKLOADS, DECODE_WORKLOADS, workload_inputs

    w = WORKLOADS[args.workload]
    seed = 1000 + list(WORKLOADS).index(args.workload) + 1
    dev = torch.device("cuda:0")
    per_set = w.tokens * w.H * (3 * 2 * w.K + (4 * w.K if w.per_dim_gate else 4) + 4)
    nsets = 3 if per_set * 3 <= 8 * 2 ** 30 else 1
    host_sets = [workload_inputs(w, seed=seed + 1000 * i) for i in range(nsets)]
    calls = []
    shared_ws = None
    for hs in host_sets:
        d = hs.to(dev)
        call = cdr.PreparedForward(d.q, d.k, d.v, d.g, d.beta, initial_state=d.initial_state,
                                   cu_seqlens=d.cu_seqlens, chunk_size=w.chunk_size,
                                   output_final_state=True, workspace=shared_ws)
        shared_ws = call.workspace
        calls.append(call)
    torch.cuda.synchronize()

    stages = (cdr.STAGE_INTRA, cdr.STAGE_CHAIN, cdr.STAGE_OUTPUT)
    names = ("intra", "chain", "output")
    # clocks: the first tens of milliseconds of GPU work run below the sustained clock, so the
    # forward runs untimed for CLOCK_WARMUP_S before the warmup steps
    tw = time.perf_counter()
    while time.perf_counter() - tw < CLOCK_WARMUP_S:
        for i in range(20):
            calls[i % nsets]()
        torch.cuda.synchronize()
    for i in range(args.warmup):
        for s in stages:
            calls[i % nsets](s)
    torch.cuda.synchronize()

    K = args.steps
    # HIP events between the kernels on every EV_STRIDE-th timed step only: an event between
    # every pair of kernels costs GPU time, which the wall-clock throughput would otherwise include
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for i in range(0, K, EV_STRIDE)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        c = calls[i % nsets]
        e = ev.get(i)
        if e is None:
            for s in stages:
                c(s)
            continue
        e[0].record()
        for j, s in enumerate(stages):
            c(s)
            e[j + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    kern_ms = {n: sum(e[j].elapsed_time(e[j + 1]) for e in ev.values()) / len(ev)
               for j, n in enumerate(names)}
    gpu_ms = sum(kern_ms.values())

    # one forward per measurement with events around it: after a 1 GiB write that pushes the
    # inputs out of the L2s and the memory-side cache (cold), and the same input set repeated
    # (warm)
    flush = torch.empty(2 ** 30 // 4, dtype=torch.float32, device=dev)

    def event_steps(n, cold):
        ts = []
        for i in range(n):
            if cold:
                flush.fill_(float(i))
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            calls[0]()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        ts.sort()
        return {"median_ms": round(ts[len(ts) // 2], 5), "min_ms": round(ts[0], 5), "steps": n}

    cold = event_steps(COLD_STEPS, True)
    warm = event_steps(COLD_STEPS, False)
    del flush

    # the same forward replayed from a captured graph (one launch per replay instead of three or
    # four): what launch overhead costs the small configurations; `value` stays the plain call
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls[0]()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        calls[0]()
    for _ in range(COLD_STEPS):
        graph.replay()
    torch.cuda.synchronize()
    ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ga.record()
    for _ in range(GRAPH_REPLAYS):
        graph.replay()
    gb.record()
    torch.cuda.synchronize()
    graph_ms = ga.elapsed_time(gb) / GRAPH_REPLAYS
    del graph

    lengths = list(w.lengths) if w.lengths is not None else [w.T] * w.B
    flops, bytes_ = kernel_work(w, lengths)
    f_nom = nominal_flops(w, lengths)
    f_min = min_flops(w, lengths)
    comp = compulsory_bytes(w, lengths)
    tokens = w.tokens
    value = tokens / (ms_step * 1e-3)
    step_tflops = f_nom / (ms_step * 1e-3) / 1e12

    per_kernel = {}
    for n in names:
        sec = kern_ms[n] * 1e-3
        tf = flops[n] / sec / 1e12
        gbs = bytes_[n] / sec / 1e9
        per_kernel[n] = {"us": round(kern_ms[n] * 1e3, 2), "tflops": round(tf, 2),
                         "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                         "mfma_busy": load_counters(n, args.workload, "sq_counters", "mfma_busy_frac")}
    # Roofline of the dominant kernel: the path is HBM-bound (its arithmetic intensity is below the
    # ridge), so the achieved figure is the forward's compulsory bytes (1540 B per token and head
    # for per-dimension gates, plus the states) over that kernel's average launch time.
    dom = max(names, key=lambda n: kern_ms[n])
    dom_s = kern_ms[dom] * 1e-3
    roof = {"bound": "hbm", "achieved": round(comp / dom_s / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = load_traffic(dom, args.workload)
    roof["kernel"] = dom
    roof["duration_us"] = round(kern_ms[dom] * 1e3, 2)
    roof["algorithmic_bytes"] = comp
    whole_step = {"hbm_gbs": round(comp / (ms_step * 1e-3) / 1e9, 1),
                  "hbm_frac": round(comp / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                  "mfma_frac_f_nom": round(step_tflops / PEAK_BF16_TFLOPS, 4),
                  "mfma_frac_f_min": round(f_min / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                  "f_nom_gflop": round(f_nom / 1e9, 3), "f_min_gflop": round(f_min / 1e9, 3),
                  "compulsory_mb": round(comp / 1e6, 2),
                  "cold_flushed": cold, "warm_same_inputs": warm,
                  "graph_replay": {"ms_per_forward": round(graph_ms, 5), "replays": GRAPH_REPLAYS,
                                   "input_sets": 1},
                  "clock_warmup_s": CLOCK_WARMUP_S}

    # parity spot check of the timed buffers against the oracle on one head, so the
    # reported number is for a forward that is correct
    spot = None
    if not args.no_cpu_baseline:
        import numpy as np
        import oracle
        hs = host_sets[(K - 1) % nsets]
        one = lambda t: None if t is None else t[:, :, :1].contiguous()  # noqa: E731
        s0 = None if hs.initial_state is None else hs.initial_state[:, :1].contiguous()
        o_ref, S_ref = oracle.recurrent_fwd(one(hs.q), one(hs.k), one(hs.v), one(hs.g), one(hs.beta),
                                            initial_state=s0, cu_seqlens=hs.cu_seqlens)
        o_gpu = calls[(K - 1) % nsets].o[:, :, :1].float().cpu().numpy()
        S_gpu = calls[(K - 1) % nsets].S[:, :1].cpu().numpy()
        spot = {"o_err_over_tol": float(np.max(np.abs(o_gpu - o_ref) / (1e-2 + 1e-2 * np.abs(o_ref)))),
                "S_err_over_tol": float(np.max(np.abs(S_gpu - S_ref) / (1e-3 + 1e-3 * np.abs(S_ref)))),
                "heads_checked": 1}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(host_sets[0], w, args.cpu_budget)

    decode = None
    if not args.no_decode:
        del calls, host_sets
        torch.cuda.empty_cache()
        decode = {n: bench_decode(n, args.steps, args.warmup) for n in DECODE_WORKLOADS}

    cp = None
    if not args.no_decode:
        cp = bench_context_parallel(args.workload, 8, args.steps, args.warmup)

    backward = None
    if not args.no_backward:
        torch.cuda.empty_cache()
        backward = bench_backward(args.workload, min(args.steps, 20), min(args.warmup, 3))

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": w.B, "T": w.T, "H": w.H, "K": w.K, "V": w.V,
                   "chunk_size": w.chunk_size, "gate": "per_dim" if w.per_dim_gate else "per_head",
                   "initial_state": w.initial_state, "output_final_state": True,
                   "lengths": list(w.lengths) if w.lengths else None, "input_sets_rotated": nsets},
        "tflops_nominal": round(step_tflops, 2),
        "mfma_frac_bf16_peak": round(step_tflops / PEAK_BF16_TFLOPS, 4),
        "gpu_ms_per_step_events": round(gpu_ms, 5),
        "whole_step": whole_step,
        "per_kernel": per_kernel,
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity_spot_check": spot,
        "decode": decode,
        "backward": backward,
        "context_parallel": cp,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
