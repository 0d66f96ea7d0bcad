#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step = one pass of the whole path on resident synthetic inputs:
  1. kda_prefill on the small-batch*heads workload: 1 sequence x T=8192
     tokens, H=8 heads, dk=dv=128, bf16 q/k/v/g/beta, FP32 initial state,
     lower_bound = -5;
  2. kda_decode at H=8 over a 4096-slot FP32 pool with 4096 scattered rows.
Each leg is bracketed by HIP events on the stream it runs on.  ``value`` is
the prefill leg's tokens*heads/s (the headline metric); ``roofline`` is the
prefill kernel against the bf16 MFMA peak; ``decode`` carries the decode
kernel's achieved HBM bandwidth against 8 TB/s.  ``cpu_baseline`` times the
FP64 oracle (test infrastructure) on the same prefill workload on the host.

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
PREFILL_BYTES_PER_TOKHEAD = 1282    # q,k,v,g (4 x 256 B) + beta (2 B) + o (256 B)
STATE_BYTES = 128 * 128 * 4
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


def cpu_baseline():
    import oracle
    from kimi_delta_attention_prefill_amd.inputs import prefill_config

    c = prefill_config(1)
    threads = min(oracle.default_threads(), c.num_seqs * c.num_heads)
    t0 = time.perf_counter()
    oracle.prefill(c.q, c.k, c.v, c.g, c.beta, c.cu_seqlens, c.scale, c.initial_state,
                   threads=threads)
    dt = time.perf_counter() - t0
    return {"value": c.total_tokens * c.num_heads / dt, "unit": "tokens*heads/s",
            "cores": threads, "kind": "oracle",
            "sample": (f"whole prefill workload ({c.num_seqs} x {c.total_tokens} tokens x "
                       f"{c.num_heads} heads), FP64 token recurrence, {dt:.2f} s wall")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-rows", type=int, default=4096)
    ap.add_argument("--decode-state", choices=["f32", "bf16"], default="f32")
    ap.add_argument("--route", choices=["auto", "serial", "chunk", "split"], default="auto")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    pc = prefill_config(1)
    to = lambda t: None if t is None else t.to(dev)
    P = dict(q=to(pc.q), k=to(pc.k), v=to(pc.v), g=to(pc.g), beta=to(pc.beta),
             cu=to(pc.cu_seqlens), s0=to(pc.initial_state))
    p_out = torch.empty_like(P["q"])
    p_fin = torch.empty_like(P["s0"])
    dt = torch.float32 if args.decode_state == "f32" else torch.bfloat16
    dc = decode_config(args.decode_rows, dt)
    D = dict(q=to(dc.q), k=to(dc.k), v=to(dc.v), g=to(dc.g), beta=to(dc.beta),
             slots=to(dc.slots), pool=to(dc.pool))
    d_out = torch.empty_like(D["q"])
    plan = kda.plan(pc.num_seqs, pc.total_tokens, pc.num_heads, pc.lower_bound, 0, route)
    ws_bytes = kda.workspace_size(pc.num_seqs, pc.total_tokens, pc.num_heads)
    p_ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        kda.prefill(P["q"], P["k"], P["v"], P["g"], P["beta"], P["cu"], scale=pc.scale,
                    lower_bound=pc.lower_bound, initial_state=P["s0"], final_state=p_fin,
                    out=p_out, workspace=p_ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        kda.decode(D["q"], D["k"], D["v"], D["g"], D["beta"], D["pool"], D["slots"],
                   scale=dc.scale, out=d_out, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    log(f"[bench] warmup {args.warmup} steps (plan {plan})")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [e[0].elapsed_time(e[1]) for e in events]
    dec_ms = [e[1].elapsed_time(e[2]) for e in events]
    pre_avg = sum(pre_ms) / len(pre_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)
    log(f"[bench] prefill {pre_avg:.4f} ms  decode {dec_avg:.4f} ms  wall/step "
        f"{1e3 * wall / args.steps:.4f} ms")

    tokheads = pc.total_tokens * pc.num_heads
    flops = tokheads * PREFILL_FLOP_PER_TOKHEAD
    pbytes = tokheads * PREFILL_BYTES_PER_TOKHEAD + 2 * pc.num_seqs * pc.num_heads * STATE_BYTES
    achieved_tf = flops / (pre_avg * 1e-3) / 1e12
    items = args.decode_rows * 8
    state_b = STATE_BYTES if args.decode_state == "f32" else STATE_BYTES // 2
    dbytes = items * (2 * state_b + DECODE_IO_BYTES_PER_ITEM)
    achieved_gbs = dbytes / (dec_avg * 1e-3) / 1e9
    route_name = {kda.ROUTE_SERIAL: "serial", kda.ROUTE_CHUNK: "chunk",
                  kda.ROUTE_SPLIT: "split"}[plan.route]

    result = {
        "metric": "KDA prefill tokens*heads/s + MFMA util; decode HBM GB/s at H=8",
        "value": tokheads / (pre_avg * 1e-3),
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
            "workload": (f"prefill 1x8192 tokens H=8 dk=dv=128 lb=-5 fp32 S0 + decode H=8 "
                         f"rows={args.decode_rows} {args.decode_state} state 4096-slot pool"),
            "prefill": {"num_seqs": pc.num_seqs, "seq_len": pc.total_tokens,
                        "num_heads": pc.num_heads, "lower_bound": pc.lower_bound,
                        "route": route_name, "dv_split": plan.dv_split,
                        "grid_blocks": plan.grid_blocks},
            "decode": {"rows": args.decode_rows, "num_heads": 8, "num_slots": 4096,
                       "state_dtype": args.decode_state},
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": f"prefill ({route_name} route)",
            "bound": "mfma", "achieved": achieved_tf, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved_tf / PEAK_BF16_TFLOPS,
            "traffic": stored_traffic(f"prefill_{route_name}_T8192_H8"),
            "algorithmic_flop_per_launch": flops,
            "algorithmic_bytes_per_launch": pbytes,
            "hbm_gbps": pbytes / (pre_avg * 1e-3) / 1e9,
            "avg_launch_ms": pre_avg,
            "us_per_chunk": 1e3 * pre_avg / ((pc.total_tokens + 31) // 32),
        },
        "decode": {
            "value": achieved_gbs, "unit": "GB/s", "avg_launch_ms": dec_avg,
            "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": PEAK_HBM_GBPS,
                         "unit": "GB/s", "frac": achieved_gbs / PEAK_HBM_GBPS,
                         "traffic": stored_traffic(
                             f"decode_{args.decode_state}_rows{args.decode_rows}_H8"),
                         "algorithmic_bytes_per_launch": dbytes},
        },
        "context": {"b200_small_bh_h8_tokheads_per_s_derived": 2.07e8,
                    "b200_prefill_speedup_vs_flashkda_geomean": 2.0512},
        "source_digest": source_digest(),
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the FP64 oracle on the host")
        result["cpu_baseline"] = cpu_baseline()
    kda.set_prefill_route(kda.ROUTE_AUTO)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
