#!/usr/bin/env python3
"""Lightning Attention benchmark on one MI355X.

One step = one ``lt_prefill`` over the M1 Lightning-layer workload: batch 1,
L = 32768 tokens, 64 heads x 128, block 256, bf16 Q/K/V, fp32 O and fp32 final
state (the block form of MiniMax Signal Lab · M1, §03, on the layer shape of
§02/§04). Inputs are seeded synthetic tensors already resident in HBM.

Prints ONE JSON line. Besides the driver's fields it carries:
  roofline      prefill kernel: algorithmic bytes per launch / mean launch
                duration (HIP events on the launch stream) against 8 TB/s HBM;
                ``traffic`` from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
                summary when it was taken on the current kernel source;
  decode        the batched decode step (256 sequences x 64 heads, 1 GiB fp32
                state updated in place), per-step HIP-event times over the run,
                state-stream GB/s against 8 TB/s;
  cpu_baseline  the fp64 oracle on the host cores, timed on the same prefill
                workload (reported baseline, not a target).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps N]
                       [--no-cpu] [--no-decode]
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

METRIC = "Lightning prefill tokens/s (H=64,d=128) + decode state GB/s, % of roofline"
HBM_PEAK_GBS = 8000.0
D = 128
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_m1_layer_L32768_traffic.json")
PREFILL_SRC = os.path.join(ROOT, "linear_attention_amd", "csrc", "prefill.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def prefill_bytes(tokens, heads, in_bytes=2, out_bytes=4, states_out=1, states_in=0):
    """Algorithmic HBM bytes of one prefill: read q, k, v once, write o once,
    write (and read) the d x d fp32 states once."""
    return tokens * heads * D * (3 * in_bytes + out_bytes) + (states_out + states_in) * heads * D * D * 4


def decode_bytes(batch, heads, in_bytes=2, out_bytes=4):
    """Algorithmic HBM bytes of one decode step: state read + write, q, k, v, o."""
    return batch * heads * (2 * D * D * 4 + 3 * D * in_bytes + D * out_bytes)


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def committed_traffic(bytes_alg):
    """Per-launch HBM traffic from the committed rocprofv3 counter summary, if it
    was taken on the current prefill kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != source_sha(PREFILL_SRC):
        return None
    return t.get("traffic_bytes_per_launch")


def run_prefill(la, torch, steps, warmup):
    import numpy as np

    import workloads

    w = workloads.M1_LAYER
    shape = (w.batch, w.seqlen, w.heads, w.head_dim)
    q, k, v = workloads.qkv_device(w.seed, shape, "bf16")
    slopes = torch.from_numpy(workloads.slopes(w.heads)).cuda()
    o = torch.empty(shape, device="cuda", dtype=torch.float32)
    st = torch.empty((w.batch, w.heads, D, D), device="cuda", dtype=torch.float32)
    stream = torch.cuda.current_stream()

    for _ in range(warmup):
        la.lt_prefill(q, k, v, slopes, w.block, o=o, state_out=st, stream=stream)
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        la.lt_prefill(q, k, v, slopes, w.block, o=o, state_out=st, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in ev]
    assert bool(torch.isfinite(o[0, -1]).all()), "non-finite prefill output"

    tokens = w.batch * w.seqlen
    ms_step = wall * 1e3 / steps
    avg_kernel_s = float(np.mean(kern_ms)) / 1e3
    bytes_alg = prefill_bytes(tokens, w.heads)
    achieved = bytes_alg / avg_kernel_s / 1e9
    traffic = committed_traffic(bytes_alg)
    return w, (q, k, v, slopes), {
        "tokens_per_s": tokens * steps / wall,
        "ms_per_step": ms_step,
        "kernel_ms_mean": avg_kernel_s * 1e3,
        "kernel_ms_min": float(np.min(kern_ms)),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "bytes_per_launch": bytes_alg,
                     "kernel": "prefill_kernel<bf16, f32>"},
    }


def run_decode(la, torch, nsteps, warmup=5):
    import numpy as np

    import workloads

    w = workloads.DECODE
    B, H = w.batch, w.heads
    # Stand-in for a 4096-token prefill state: Gaussian with the stationary
    # per-head scale of the state recurrence for unit-variance-over-128 inputs.
    # The kernel's time does not depend on the values; the parity tests use
    # oracle-prefill states.
    s = torch.from_numpy(workloads.slopes(H)).double()
    lam2 = torch.exp(-2 * s)
    std = torch.sqrt((1 - lam2 ** w.extra["history"]) / (1 - lam2)) / D
    state = workloads.state_device(w.seed, (B, H, D, D), std=1.0)
    state.mul_(std.float().cuda().view(1, H, 1, 1))
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed + 1)
    qkv = (torch.randn((nsteps + warmup, 3, B, H, D), generator=g, device="cuda")
           .mul_(workloads.INPUT_SCALE).to(torch.bfloat16))
    slopes = torch.from_numpy(workloads.slopes(H)).cuda()
    o = torch.empty((B, H, D), device="cuda", dtype=torch.float32)
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        la.lt_decode(qkv[i, 0], qkv[i, 1], qkv[i, 2], slopes, state, o=o, stream=stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(nsteps)]
    for i, (a, b) in enumerate(ev):
        x = qkv[warmup + i]
        a.record(stream)
        la.lt_decode(x[0], x[1], x[2], slopes, state, o=o, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    assert bool(torch.isfinite(o).all()), "non-finite decode output"
    med = float(np.median(ms))
    nbytes = decode_bytes(B, H)
    gbs = nbytes / (med / 1e3) / 1e9
    return {
        "workload": w.name, "batch": B, "heads": H, "head_dim": D, "steps": nsteps,
        "steps_per_s": round(1e3 / med, 1),
        "ms_per_step_median": round(med, 5),
        "ms_per_step_p10": round(float(np.percentile(ms, 10)), 5),
        "ms_per_step_p90": round(float(np.percentile(ms, 90)), 5),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": nbytes, "kernel": "decode_kernel<bf16, f32>"},
        "state": "Gaussian stand-in with the per-head scale of a 4096-token prefill state",
    }


def run_cpu_baseline(w, dev_inputs, tokens):
    """The fp64 oracle (as it stands) on the host cores, on the first `tokens`
    tokens of the same prefill inputs, all heads."""
    import oracle

    q, k, v, slopes = dev_inputs
    hq, hk, hv = (x[:, :tokens].float().cpu().numpy() for x in (q, k, v))
    sl = slopes.cpu().numpy()
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.recurrence_batch(hq, hk, hv, sl)
    dt = time.perf_counter() - t0
    return {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {tokens} of {w.seqlen} tokens, all {w.heads} heads "
                      f"({tokens * w.heads} (token, head) pairs, {dt:.2f} s, fp64)",
            "host_cpus": len(os.sched_getaffinity(0))}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--cpu-tokens", type=int, default=32768)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(heads and sequences are independent, so each GPU would take its own heads).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    import linear_attention_amd as la

    log("[bench] prefill m1_layer L=32768 H=64 d=128 block=256")
    w, dev_inputs, pre = run_prefill(la, torch, args.steps, args.warmup)
    log(f"[bench] prefill {pre['kernel_ms_mean']:.3f} ms/launch")
    dec = None
    if not args.no_decode:
        log(f"[bench] decode batch=256 H=64, {args.decode_steps} steps")
        dec = run_decode(la, torch, args.decode_steps)
        log(f"[bench] decode {dec['ms_per_step_median']:.4f} ms/step")
    cpu = None
    if not args.no_cpu:
        log(f"[bench] cpu oracle on {args.cpu_tokens} tokens")
        cpu = run_cpu_baseline(w, dev_inputs, min(args.cpu_tokens, w.seqlen))

    line = {
        "metric": METRIC,
        "value": round(pre["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen, "heads": w.heads,
                   "head_dim": w.head_dim, "block": w.block, "in_dtype": "bf16",
                   "out_dtype": "f32", "state_out": "f32"},
        "roofline": pre["roofline"],
        "kernel_ms_mean": round(pre["kernel_ms_mean"], 5),
        "decode": dec,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
