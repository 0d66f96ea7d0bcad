#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step = one pass of the whole path on resident synthetic inputs:
  1. the prefill of the small-batch*heads workload: 1 sequence x T=8192
     tokens, H=8 heads, dk=dv=128, bf16 q/k/v/g/beta, FP32 initial state,
     lower_bound = -5.  With the two-pass route (the one chosen for this
     shape) it runs as kda_prefill_prepare + kda_prefill_chain, the same two
     kernels kda_prefill launches, so that each kernel can be timed;
  2. kda_decode at H=8 over a 4096-slot FP32 pool with 4096 scattered rows.
Every call is bracketed by HIP events on the stream it runs on.  ``value``
is the prefill's tokens*heads/s (the headline metric); ``roofline`` is the
preparation kernel (the longest single prefill kernel; the chain pass is
three launches when one long sequence is cut into windows, reported under
``prefill.kernels.chain_pass``) against its roofline; ``decode``
carries the decode kernel's HBM bandwidth against 8 TB/s and against a
device-to-device copy timed in the same run.  ``prefill.cold_cache`` repeats the
prefill with a 512 MiB write before each call (outside the timed region), so
that its inputs start in HBM rather than in the last-level cache.
``cpu_baseline`` times the
FP64 oracle (test infrastructure) on the same prefill workload on the host.
After the timed steps, ``decode_sweep`` times kda_decode at rows 1 ... 4096
(FP32 and BF16 pools), ``multitoken_decode_sweep`` the T = 2, 4, 8 multi-token
decode through kda_prefill_pool_ex, and ``configs`` prefill configurations 2
(16 varlen sequences, H=32) and 3 (4 x 8192, H=64) with their kernel's MFMA
and HBM fractions.

Prints one JSON line on stdout; progress goes to stderr.
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

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PREFILL_FLOP_PER_TOKHEAD = 131072   # 8 * dk * dv: Akk, Mqk, [Kg;Qg]S, T V', [Kr^T;Mqk]U
# Split of those FLOPs between the two kernels of the two-pass route:
# preparation = Akk + Mqk + T V' (3 x 32 x 128 MAC per token*head),
# chain = [Kg;Qg] S (64 x 128 x 128 / 32) + the fused [S;O] update (160 x 128).
PREP_FLOP_PER_TOKHEAD = 24576
CHAIN_FLOP_PER_TOKHEAD = 106496
PREFILL_BYTES_PER_TOKHEAD = 1282    # q,k,v,g (4 x 256 B) + beta (2 B) + o (256 B)
PREP_BYTES_PER_TOKHEAD = 1026       # the preparation pass reads q,k,v,g,beta
STATE_BYTES = 128 * 128 * 4
COLD_FLUSH_BYTES = 512 << 20        # written before each cold-cache prefill call
DECODE_IO_BYTES_PER_ITEM = 1282


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kimi_delta_attention_prefill_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, or None
    when the summary is missing or was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest():
        return None
    return rec.get("bytes_per_launch")


def stored_mfma(workload: str):
    """Per-kernel MFMA counters (busy % of SIMDs, executed MFMA TFLOP/s) from a
    committed rocprofv3 --pmc summary, or {} when missing or stale."""
    path = os.path.join(ROOT, "profiles", f"mfma_{workload}.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest():
        return {}
    return rec.get("kernels", {})


def stats(ms):
    a = sorted(ms)
    pick = lambda f: a[min(len(a) - 1, max(0, int(round(f * (len(a) - 1)))))]
    return {"median_ms": pick(0.5), "p10_ms": pick(0.1), "p90_ms": pick(0.9),
            "mean_ms": sum(a) / len(a)}


def copy_bandwidth(torch, dev, nbytes=1 << 30, reps=5):
    """Device-to-device copy GB/s (read + write) on the same GPU and stream."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps * 1e-3
    del src, dst
    return 2 * nbytes / t / 1e9


def decode_sweep(torch, dev, kda, copy_gbs, steps=30, warmup=5):
    """kda_decode at H=8 for rows 1, 2, 4, ..., 4096 over a 4096-slot pool, FP32
    and BF16 states: time per call over `steps` calls replayed from a graph, achieved
    GB/s (state read + write and the row inputs/outputs) and its fraction of
    the same run's device copy."""
    from kimi_delta_attention_prefill_amd.inputs import decode_config, make_decode_case

    out = []
    for dt, name, state_b in ((torch.float32, "f32", STATE_BYTES),
                              (torch.bfloat16, "bf16", STATE_BYTES // 2)):
        pool = decode_config(1, dt).pool.to(dev)       # the 4096-slot pool of the workload
        rows = 1
        while rows <= 4096:
            d = make_decode_case(rows, 8, 4096, dt, seed=20264 + rows, with_pool=False)
            to = lambda t: t.to(dev)
            args = (to(d.q), to(d.k), to(d.v), to(d.g), to(d.beta), pool, to(d.slots))
            o = torch.empty_like(args[0])
            for _ in range(warmup):
                kda.decode(*args, scale=d.scale, out=o)
            # `steps` calls captured in one graph and replayed between one pair
            # of events, as a serving loop would issue them: an event-bracketed
            # call of a few microseconds, or calls launched one by one from
            # Python, mostly time the launches themselves
            graph = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.graph(graph):
                for _ in range(steps):
                    kda.decode(*args, scale=d.scale, out=o)
            graph.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            del graph
            gbs = rows * 8 * (2 * state_b + DECODE_IO_BYTES_PER_ITEM) / (ms * 1e-3) / 1e9
            out.append({"state": name, "rows": rows, "ms_per_call": ms,
                        "gbps": gbs, "frac_of_peak": gbs / PEAK_HBM_GBPS,
                        "frac_of_copy": gbs / copy_gbs})
            log(f"[bench] decode sweep {name} rows={rows} {ms * 1e3:.1f} us {gbs:.0f} GB/s")
            rows *= 2
        del pool
    return out


def multitoken_sweep(torch, dev, kda, copy_gbs, steps=10, warmup=3):
    """Multi-token decode (T = 2, 4, 8 new tokens per row) through
    kda_prefill_pool_ex at H=8 over a 4096-slot pool (FP32 and BF16), rows 1,
    64 and 4096, with the decode front-end (softplus gates, beta logits,
    q/k L2 norm): time per call over graph-replayed calls and GB/s of state
    read + write plus the tokens' inputs and outputs."""
    from kimi_delta_attention_prefill_amd.inputs import decode_config, make_prefill_raw_case

    fe = kda.FrontEnd(gate_mode=kda.GATE_SOFTPLUS, beta_logits=True, normalize_qk=True,
                      norm_eps=1e-6)
    out = []
    for dt, name, state_b in ((torch.float32, "f32", STATE_BYTES),
                              (torch.bfloat16, "bf16", STATE_BYTES // 2)):
        pool = decode_config(1, dt).pool.to(dev)
        for tokens in (2, 4, 8):
            for rows in (1, 64, 4096):
                c = make_prefill_raw_case([tokens] * rows, 8, init_std=None,
                                          seed=30000 + rows + tokens)
                gen = torch.Generator().manual_seed(30001 + rows)
                slots = torch.randperm(4096, generator=gen)[:rows].to(torch.int32).to(dev)
                x = [t.to(dev) for t in (c.q, c.k, c.v, c.g, c.beta, c.cu_seqlens)]
                o = torch.empty_like(x[0])
                ws_bytes = kda.workspace_size(rows, rows * tokens, 8)
                ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
                call = lambda: kda.prefill_pool(*x, slots, pool, scale=c.scale,
                                                lower_bound=float("-inf"), out=o, workspace=ws,
                                                frontend=fe)
                for _ in range(warmup):
                    call()
                graph = torch.cuda.CUDAGraph()
                torch.cuda.synchronize()
                with torch.cuda.graph(graph):
                    for _ in range(steps):
                        call()
                graph.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                graph.replay()
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / steps
                del graph
                nbytes = rows * 8 * (2 * state_b + tokens * PREFILL_BYTES_PER_TOKHEAD)
                gbs = nbytes / (ms * 1e-3) / 1e9
                out.append({"state": name, "tokens": tokens, "rows": rows, "ms_per_call": ms,
                            "gbps": gbs, "frac_of_peak": gbs / PEAK_HBM_GBPS,
                            "frac_of_copy": gbs / copy_gbs,
                            "route": kda.plan(rows, rows * tokens, 8, float("-inf"), 0,
                                              kda.ROUTE_AUTO).route})
                log(f"[bench] multi-token decode {name} T={tokens} rows={rows} "
                    f"{ms * 1e3:.1f} us {gbs:.0f} GB/s")
        del pool
    return out


def fused_configs(torch, dev, kda, configs=(2, 3), steps=10, warmup=3):
    """Prefill configurations 2 (16 varlen sequences, H=32) and 3 (4 x 8192,
    H=64, lb=-8) on the route the planner picks (the fused chunk kernel, one
    launch per call): event-timed calls, tokens*heads/s, and the kernel's
    MFMA and HBM fractions from the algorithmic FLOPs and bytes."""
    from kimi_delta_attention_prefill_amd.inputs import prefill_config

    res = {}
    stream = torch.cuda.current_stream()
    for i in configs:
        log(f"[bench] prefill configuration {i}")
        c = prefill_config(i)
        x = [t.to(dev) for t in (c.q, c.k, c.v, c.g, c.beta, c.cu_seqlens)]
        s0 = None if c.initial_state is None else c.initial_state.to(dev)
        N, T, H = c.num_seqs, c.total_tokens, c.num_heads
        plan = kda.plan(N, T, H, c.lower_bound, 0, kda.ROUTE_AUTO)
        o = torch.empty_like(x[0])
        fin = torch.empty((N, H, 128, 128), dtype=torch.float32, device=dev)
        ws_bytes = kda.workspace_size(N, T, H)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
        call = lambda: kda.prefill(*x, scale=c.scale, lower_bound=c.lower_bound,
                                   initial_state=s0, final_state=fin, out=o, workspace=ws,
                                   stream=stream)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for e in ev:
            e[0].record(stream)
            call()
            e[1].record(stream)
        torch.cuda.synchronize()
        st = stats([e[0].elapsed_time(e[1]) for e in ev])
        tokheads = T * H
        t = st["mean_ms"] * 1e-3
        flops = tokheads * PREFILL_FLOP_PER_TOKHEAD
        nbytes = tokheads * PREFILL_BYTES_PER_TOKHEAD + (N * H * STATE_BYTES) * (
            2 if s0 is not None else 1)
        route = {kda.ROUTE_SERIAL: "serial", kda.ROUTE_CHUNK: "chunk",
                 kda.ROUTE_SPLIT: "split"}[plan.route]
        kname = f"prefill_{route}"
        res[f"config{i}"] = dict(
            st, workload=(f"prefill {N} sequence(s), {T} tokens, H={H}, dk=dv=128, "
                          f"lb={c.lower_bound:g}, {'fp32' if s0 is not None else 'zero'} S0"),
            route=route, tokheads_per_s=tokheads / t,
            mfma_tflops=flops / t / 1e12, mfma_frac=flops / t / 1e12 / PEAK_BF16_TFLOPS,
            hbm_gbps=nbytes / t / 1e9, hbm_frac=nbytes / t / 1e9 / PEAK_HBM_GBPS,
            algorithmic_flop_per_call=flops, algorithmic_bytes_per_call=nbytes,
            kernels={kname: dict(st, launches_per_call=1,
                                 traffic=stored_traffic(f"{kname}_T{T}_H{H}"),
                                 mfma_counters=stored_mfma(f"{kname}_T{T}_H{H}").get(
                                     f"{kname}_kernel"))})
        log(f"[bench] configuration {i}: {st['mean_ms']:.3f} ms, "
            f"{tokheads / t:.3e} tokens*heads/s")
        del x, s0, o, fin, ws
    return res


def cpu_baseline(config=1, min_seconds=10.0, max_runs=50):
    """The FP64 oracle on the whole prefill workload, repeated until about
    `min_seconds` of wall time have passed; reports the mean rate."""
    import oracle
    from kimi_delta_attention_prefill_amd.inputs import prefill_config

    c = prefill_config(config)
    threads = min(oracle.default_threads(), c.num_seqs * c.num_heads)
    runs, t0 = 0, time.perf_counter()
    while runs < max_runs and (runs == 0 or time.perf_counter() - t0 < min_seconds):
        oracle.prefill(c.q, c.k, c.v, c.g, c.beta, c.cu_seqlens, c.scale, c.initial_state,
                       threads=threads)
        runs += 1
    dt = (time.perf_counter() - t0) / runs
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f
                              if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": c.total_tokens * c.num_heads / dt, "unit": "tokens*heads/s",
            "cores": threads, "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model,
            "kind": "oracle",
            "sample": (f"whole prefill workload ({c.num_seqs} sequence(s), {c.total_tokens} "
                       f"tokens in all, {c.num_heads} heads), FP64 token recurrence, {runs} runs, "
                       f"{dt:.3f} s wall each on {threads} threads")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-rows", type=int, default=4096)
    ap.add_argument("--decode-state", choices=["f32", "bf16"], default="f32")
    ap.add_argument("--route", choices=["auto", "serial", "chunk", "split"], default="auto")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-sweep", action="store_true",
                    help="skip the kda_decode sweep over rows 1, 2, ..., 4096 (FP32 and BF16 "
                         "pools) and the multi-token (T = 2, 4, 8) decode sweep")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip prefill configurations 2 and 3 (reported under 'configs')")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="prefill calls timed after a 512 MiB write has flushed the caches "
                         "(0 = skip)")
    ap.add_argument("--prefill-config", type=int, choices=[0, 1, 2, 3], default=1,
                    help="prefill workload: 1 (default) = 1 x 8192 x H=8, the headline; "
                         "0 = 1 x 64 x H=2; 2 = 16 varlen x H=32; 3 = 4 x 8192 x H=64, lb=-8")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the KDA path needs no cross-GPU exchange and "
              "this build runs on a single MI355X; use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import kimi_delta_attention_prefill_amd as kda
    from kimi_delta_attention_prefill_amd.inputs import decode_config, prefill_config

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kda.load()
    route = {"auto": kda.ROUTE_AUTO, "serial": kda.ROUTE_SERIAL, "chunk": kda.ROUTE_CHUNK,
             "split": kda.ROUTE_SPLIT}[args.route]
    kda.set_prefill_route(route)

    log("[bench] generating inputs")
    pc = prefill_config(args.prefill_config)
    tag = f"T{pc.total_tokens}_H{pc.num_heads}"
    to = lambda t: None if t is None else t.to(dev)
    P = dict(q=to(pc.q), k=to(pc.k), v=to(pc.v), g=to(pc.g), beta=to(pc.beta),
             cu=to(pc.cu_seqlens), s0=to(pc.initial_state))
    p_out = torch.empty_like(P["q"])
    p_fin = torch.empty((pc.num_seqs, pc.num_heads, 128, 128), dtype=torch.float32, device=dev)
    dt = torch.float32 if args.decode_state == "f32" else torch.bfloat16
    dc = decode_config(args.decode_rows, dt)
    D = dict(q=to(dc.q), k=to(dc.k), v=to(dc.v), g=to(dc.g), beta=to(dc.beta),
             slots=to(dc.slots), pool=to(dc.pool))
    d_out = torch.empty_like(D["q"])
    plan = kda.plan(pc.num_seqs, pc.total_tokens, pc.num_heads, pc.lower_bound, 0, route)
    two_pass = plan.route == kda.ROUTE_SPLIT
    ws_bytes = kda.workspace_size(pc.num_seqs, pc.total_tokens, pc.num_heads)
    if two_pass:
        ws_bytes = kda.records_size(pc.num_seqs, pc.total_tokens, pc.num_heads)
    p_ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    stream = torch.cuda.current_stream()

    def prefill_call(ev=None):
        rec = (lambda i: ev[i].record(stream)) if ev is not None else (lambda i: None)
        rec(0)
        if two_pass:
            kda.prefill_prepare(P["q"], P["k"], P["v"], P["g"], P["beta"], P["cu"],
                                lower_bound=pc.lower_bound, records=p_ws, stream=stream)
            rec(1)
            kda.prefill_chain(p_ws, P["cu"], pc.num_heads, scale=pc.scale,
                              total_tokens=pc.total_tokens, initial_state=P["s0"],
                              final_state=p_fin, out=p_out, stream=stream)
        else:
            kda.prefill(P["q"], P["k"], P["v"], P["g"], P["beta"], P["cu"], scale=pc.scale,
                        lower_bound=pc.lower_bound, initial_state=P["s0"], final_state=p_fin,
                        out=p_out, workspace=p_ws, stream=stream)
            rec(1)
        rec(2)

    def step(ev=None):
        rec = (lambda i: ev[i].record(stream)) if ev is not None else (lambda i: None)
        prefill_call(ev)
        kda.decode(D["q"], D["k"], D["v"], D["g"], D["beta"], D["pool"], D["slots"],
                   scale=dc.scale, out=d_out, stream=stream)
        rec(3)

    log(f"[bench] warmup {args.warmup} steps (plan {plan})")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [e[0].elapsed_time(e[2]) for e in events]
    k1_ms = [e[0].elapsed_time(e[1]) for e in events]
    k2_ms = [e[1].elapsed_time(e[2]) for e in events]
    dec_ms = [e[2].elapsed_time(e[3]) for e in events]
    pre, dec = stats(pre_ms), stats(dec_ms)
    log(f"[bench] prefill {pre['mean_ms']:.4f} ms  decode {dec['mean_ms']:.4f} ms  "
        f"wall/step {1e3 * wall / args.steps:.4f} ms")
    # Cold-cache prefill: a 512 MiB write before each call evicts the inputs
    # from L2 and the last-level cache (the flush is outside the timed region).
    cold = None
    if args.cold_steps > 0:
        log(f"[bench] timing {args.cold_steps} cold-cache prefill calls")
        flush = torch.empty(COLD_FLUSH_BYTES, dtype=torch.uint8, device=dev)
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
               for _ in range(args.cold_steps)]
        for i in range(args.cold_steps):
            flush.fill_(i & 0xFF)
            prefill_call(cev[i])
        torch.cuda.synchronize()
        cold = dict(stats([e[0].elapsed_time(e[2]) for e in cev]),
                    flush_bytes=COLD_FLUSH_BYTES)
        if two_pass:
            cold["kernels"] = {"prefill_split_prep": stats([e[0].elapsed_time(e[1]) for e in cev]),
                               "chain_pass": stats([e[1].elapsed_time(e[2]) for e in cev])}
        del flush
    log("[bench] timing a device-to-device copy")
    copy_gbs = copy_bandwidth(torch, dev)

    tokheads = pc.total_tokens * pc.num_heads
    chunks = (pc.total_tokens + 31) // 32
    flops = tokheads * PREFILL_FLOP_PER_TOKHEAD
    pbytes = tokheads * PREFILL_BYTES_PER_TOKHEAD + 2 * pc.num_seqs * pc.num_heads * STATE_BYTES
    items = args.decode_rows * 8
    state_b = STATE_BYTES if args.decode_state == "f32" else STATE_BYTES // 2
    dbytes = items * (2 * state_b + DECODE_IO_BYTES_PER_ITEM)
    achieved_gbs = dbytes / (dec["mean_ms"] * 1e-3) / 1e9
    route_name = {kda.ROUTE_SERIAL: "serial", kda.ROUTE_CHUNK: "chunk",
                  kda.ROUTE_SPLIT: "split"}[plan.route]
    units = pc.num_seqs * pc.num_heads

    kernels = {}
    if two_pass:
        k1, k2 = stats(k1_ms), stats(k2_ms)
        prep_tf = tokheads * PREP_FLOP_PER_TOKHEAD / (k1["mean_ms"] * 1e-3) / 1e12
        prep_gbs = tokheads * PREP_BYTES_PER_TOKHEAD / (k1["mean_ms"] * 1e-3) / 1e9
        chain_tf = tokheads * CHAIN_FLOP_PER_TOKHEAD / (k2["mean_ms"] * 1e-3) / 1e12
        kernels["prefill_split_prep"] = dict(
            k1, bound="hbm", achieved=prep_gbs, peak=PEAK_HBM_GBPS, unit="GB/s",
            frac=prep_gbs / PEAK_HBM_GBPS, traffic=stored_traffic(f"prefill_split_prep_{tag}"),
            algorithmic_bytes_per_launch=tokheads * PREP_BYTES_PER_TOKHEAD,
            algorithmic_flop_per_launch=tokheads * PREP_FLOP_PER_TOKHEAD, mfma_tflops=prep_tf)
        windows = plan.windows
        launches = (["prefill_split_window_a", "prefill_split_window_c"]
                    if windows > 1 else ["prefill_split_chain"])
        counters = stored_mfma(
            f"prefill_split_{tag}_decode_rows{args.decode_rows}_{args.decode_state}")
        if "prefill_split_prep" in counters:
            kernels["prefill_split_prep"]["mfma_counters"] = counters["prefill_split_prep"]
        serial_steps = (2 * plan.window_chunks if windows > 1 else chunks)
        kernels["chain_pass"] = dict(
            k2, launches=launches, bound="mfma", achieved=chain_tf, peak=PEAK_BF16_TFLOPS,
            unit="TFLOP/s", frac=chain_tf / PEAK_BF16_TFLOPS,
            algorithmic_flop_per_call=tokheads * CHAIN_FLOP_PER_TOKHEAD,
            windows=windows, window_chunks=plan.window_chunks,
            serial_chunk_steps=serial_steps,
            us_per_serial_chunk_step=1e3 * k2["mean_ms"] / serial_steps,
            mfma_counters={k: counters[k] for k in launches if k in counters} or None)
        # The roofline names the longest single kernel that bench times on its own:
        # the preparation (the chain pass is several launches).
        dom = "prefill_split_prep"
    else:
        dom = f"prefill_{route_name}"
        tf = flops / (pre["mean_ms"] * 1e-3) / 1e12
        kernels[dom] = dict(pre, bound="mfma", achieved=tf, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                            frac=tf / PEAK_BF16_TFLOPS,
                            traffic=stored_traffic(f"{dom}_{tag}"),
                            algorithmic_flop_per_launch=flops)
    d = kernels[dom]
    roofline = {"kernel": dom, "bound": d["bound"], "achieved": d["achieved"], "peak": d["peak"],
                "unit": d["unit"], "frac": d["frac"], "traffic": d["traffic"],
                "avg_launch_ms": d["mean_ms"], "median_launch_ms": d["median_ms"],
                "scope": ("prefill, the headline metric (longest single prefill kernel); the "
                          "decode kernel, the step's longest, is under decode.roofline")}
    for key in ("algorithmic_flop_per_launch", "algorithmic_bytes_per_launch", "mfma_tflops"):
        if key in d:
            roofline[key] = d[key]

    result = {
        "metric": "KDA prefill tokens*heads/s + MFMA util; decode HBM GB/s at H=8",
        "value": tokheads / (pre["mean_ms"] * 1e-3),
        "unit": "tokens*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * wall / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"prefill {pc.num_seqs} sequence(s), {pc.total_tokens} tokens, "
                         f"H={pc.num_heads}, dk=dv=128, lb={pc.lower_bound:g}, "
                         f"{'fp32' if pc.initial_state is not None else 'zero'} S0 + decode H=8 "
                         f"rows={args.decode_rows} {args.decode_state} state 4096-slot pool"),
            "prefill": {"num_seqs": pc.num_seqs, "seq_len": pc.total_tokens,
                        "num_heads": pc.num_heads, "lower_bound": pc.lower_bound,
                        "route": route_name, "dv_split": plan.dv_split,
                        "grid_blocks": plan.grid_blocks},
            "decode": {"rows": args.decode_rows, "num_heads": 8, "num_slots": 4096,
                       "state_dtype": args.decode_state},
            "parallelism": "single GPU",
        },
        "roofline": roofline,
        "prefill": dict(pre, tokheads_per_s=tokheads / (pre["mean_ms"] * 1e-3),
                        mfma_tflops=flops / (pre["mean_ms"] * 1e-3) / 1e12,
                        mfma_frac=flops / (pre["mean_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                        algorithmic_flop_per_call=flops, algorithmic_bytes_per_call=pbytes,
                        hbm_gbps=pbytes / (pre["mean_ms"] * 1e-3) / 1e9,
                        us_per_chunk=1e3 * pre["mean_ms"] / chunks, kernels=kernels,
                        cold_cache=(None if cold is None else dict(
                            cold, tokheads_per_s=tokheads / (cold["mean_ms"] * 1e-3)))),
        "decode": dict(dec, value=achieved_gbs, unit="GB/s",
                       copy_gbps_same_run=copy_gbs, frac_of_copy=achieved_gbs / copy_gbs,
                       roofline={"bound": "hbm", "achieved": achieved_gbs,
                                 "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                 "frac": achieved_gbs / PEAK_HBM_GBPS,
                                 "traffic": stored_traffic(
                                     f"decode_{args.decode_state}_rows{args.decode_rows}_H8"),
                                 "algorithmic_bytes_per_launch": dbytes}),
        "context": {"b200_small_bh_h8_tokheads_per_s_derived": 2.07e8,
                    "b200_prefill_speedup_vs_flashkda_geomean": 2.0512},
        "source_digest": source_digest(),
    }
    if not args.no_decode_sweep:
        del D, d_out
        result["decode_sweep"] = decode_sweep(torch, dev, kda, copy_gbs)
        result["multitoken_decode_sweep"] = multitoken_sweep(torch, dev, kda, copy_gbs)
    if not args.no_configs:
        del P, p_out, p_fin, p_ws
        result["configs"] = fused_configs(torch, dev, kda)
    if not args.no_cpu_baseline:
        log("[bench] timing the FP64 oracle on the host")
        result["cpu_baseline"] = cpu_baseline(args.prefill_config)
    kda.set_prefill_route(kda.ROUTE_AUTO)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
