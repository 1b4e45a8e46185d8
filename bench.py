#!/usr/bin/env python3
"""Lightning Attention benchmark on one MI355X.

One step = one ``lt_prefill`` over the M1 Lightning-layer workload: batch 1,
L = 32768 tokens, 64 heads x 128, block 256, bf16 Q/K/V, fp32 O and fp32 final
state (the block form of MiniMax Signal Lab · M1, §03, on the layer shape of
§02/§04). Inputs are seeded synthetic tensors already resident in HBM.

Prints ONE JSON line. Besides the standard fields (metric, value, unit, steps, config ...) it carries:
  roofline      the prefill call: algorithmic bytes per call / mean call time
                (HIP events on the launch stream) against 8 TB/s HBM;
                ``traffic``: HBM bytes per call from the committed rocprofv3
                FETCH_SIZE/WRITE_SIZE summary when it was taken on the current
                library sources, else null;
  configs       every other workload of the benchmark set, each with its own
                roofline and oracle baseline: the tiny fp32 prefill, the
                1M-token prefill, the 16-sequence varlen prefill with carried
                states, and a packed batch of 2 x 131072 tokens beside
                lt_prefill on the same shape;
  decode        the batched decode step (256 sequences x 64 heads, 1 GiB fp32
                state updated in place), per-step HIP-event times over the run,
                state-stream GB/s against 8 TB/s, with counter traffic;
  norm_gate     the same prefill and decode with the normalisation and gate
                fused into the epilogue (bf16 gate, bf16 y);
  backward      lt_prefill_backward (dq, dk, dv, dS0) on the M1 layer and on a
                4 x 8192-token batch of the same heads, with counter traffic;
  softmax       the hybrid's softmax attention layer (§02: 64 query / 8 K/V
                heads, partial RoPE): causal prefill of 32768 tokens against the
                bf16 MFMA peak, and a 16 x 32768-token KV-cache decode step
                against HBM;
  cpu_baseline  the fp64 oracle on the host cores, timed on a bounded sample of
                the same prefill workload (reported baseline, not a target).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps N]
                       [--no-cpu] [--no-configs] [--no-decode] [--no-norm-gate]
                       [--no-backward] [--no-softmax] [--no-slopes-scaled] [--no-settle]
       python bench.py --only WORKLOAD --steps K --warmup W
                       (one workload alone, for profiler passes: m1_layer,
                        decode, backward, tiny_f32, long_1m, varlen, varlen_2x131072)
       python bench.py --copy-calibration BYTES     (plain device copy, for
                                                     rocprofv3 counter scaling)
       python bench.py --traffic-from COPY_DIR FETCH_DIR WRITE_DIR --traffic-workload NAME --calls N
                       (turn rocprofv3 --pmc CSV runs of `--only NAME` into the
                        per-call HBM traffic entry in profiles/traffic_counters.json)
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Lightning prefill tokens/s (H=64,d=128) + decode state GB/s, % of roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0
D = 128
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def prefill_bytes(tokens, heads, in_bytes=2, out_bytes=4, states_out=1, states_in=0):
    """Algorithmic HBM bytes of one prefill: read q, k, v once, write o once,
    write (and read) the d x d fp32 states once."""
    return tokens * heads * D * (3 * in_bytes + out_bytes) + (states_out + states_in) * heads * D * D * 4


def decode_bytes(batch, heads, in_bytes=2, out_bytes=4):
    """Algorithmic HBM bytes of one decode step: state read + write, q, k, v, o."""
    return batch * heads * (2 * D * D * 4 + 3 * D * in_bytes + D * out_bytes)


def backward_bytes(batch, seqlen, heads, grad_bytes=4):
    """q, k, v, dO read once and dq, dk, dv written once, plus dS read and dS0 written."""
    return batch * seqlen * heads * D * (4 * 2 + 3 * grad_bytes) + 2 * batch * heads * D * D * 4


# The library sources each profiled workload runs (kernels, launch plan and
# the ABI): a counter summary is valid while these files are unchanged.
_CSRC = os.path.join(ROOT, "linear_attention_amd", "csrc")
_COMMON = [os.path.join(_CSRC, f) for f in ("lightning_api.cpp", "internal.h")] + \
    [os.path.join(ROOT, "include", "lightning.h")]
_PREFILL = _COMMON + [os.path.join(_CSRC, f) for f in ("prefill_heads.hip", "tiles.h")]
WORKLOAD_SRCS = {
    "m1_layer": _PREFILL, "long_1m": _PREFILL, "varlen": _PREFILL, "varlen_2x131072": _PREFILL,
    "tiny_f32": _COMMON + [os.path.join(_CSRC, "prefill_slices.hip")],
    "decode": _COMMON + [os.path.join(_CSRC, "decode.hip")],
    "backward_b1_L32768": _PREFILL + [os.path.join(_CSRC, "backward.hip")],
    "backward_b4_L8192": _PREFILL + [os.path.join(_CSRC, "backward.hip")],
}


def sources_hash(workload):
    import hashlib

    h = hashlib.sha256()
    for path in WORKLOAD_SRCS[workload]:
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(workload):
    """Per-call HBM traffic of `workload` from the committed rocprofv3 counter
    summary, if it was taken on the current sources of that workload; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            entry = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not entry or entry.get("sources_hash") != sources_hash(workload):
        return None
    return entry.get("traffic_bytes_per_call")


_SETTLE = {"on": True, "x": None}


def settle_gpu(torch):
    """About 30 ms of bf16 matrix products (hipBLASLt, nothing of this library)
    before a timed workload. After the GPU has been idle, the first tens of
    milliseconds of back-to-back work run in a slower state: M1-layer prefill
    calls 6-25 of a burst after 0.5 s idle took 0.561-0.566 ms against 0.500 ms
    once settled, and 0.495 ms from the first call on after these products (or
    after 20 GB of plain copies). The timed region is unchanged: exactly
    `steps` calls after `warmup` untimed ones. --no-settle turns it off."""
    if not _SETTLE["on"]:
        return
    if _SETTLE["x"] is None:
        g = torch.Generator(device="cuda")
        g.manual_seed(7)
        _SETTLE["x"] = torch.randn((8192, 8192), device="cuda", dtype=torch.bfloat16, generator=g)
    x = _SETTLE["x"]
    for _ in range(40):
        y = x @ x
    torch.cuda.synchronize()
    del y


def time_calls(torch, call, steps, warmup, stream):
    """Mean and median call time (ms) from HIP events recorded on `stream` around
    each of `steps` calls after `warmup` untimed ones (and settle_gpu before
    them), and the wall time (s) of the timed calls bracketed by device
    synchronisations. Python's garbage collector is off from the settling work
    to the end of the timed calls (as in the standard library's timeit), so
    that a collection pass cannot stall the host between two launches; the
    collection before it runs ahead of settle_gpu, since an idle gap of tens
    of milliseconds after it puts the GPU back into its slower state."""
    import gc

    import numpy as np

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    was_on = gc.isenabled()
    gc.collect()
    gc.disable()
    try:
        settle_gpu(torch)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for a, b in ev:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    finally:
        if was_on:
            gc.enable()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    return float(ms.mean()), float(np.median(ms)), ms, wall


def hbm_roofline(nbytes, ms, kernel, traffic=None):
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "bytes_per_launch": int(nbytes),
            "kernel": kernel}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_build():
    import oracle

    flags = [a for a in oracle.GCC_CMD if a.startswith("-O") or a.startswith("-m") or a.startswith("-f")]
    return "gcc " + " ".join(flags) + " (portable build for the GPU host; not -march=native)"


def oracle_rate(run, units_per_run, min_seconds, max_reps=50):
    """Repeats run() until min_seconds of host time; returns (units/s, reps, seconds)."""
    reps, dt = 0, 0.0
    while reps < max_reps and (reps == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        run()
        dt += time.perf_counter() - t0
        reps += 1
    return units_per_run * reps / dt, reps, dt


def blas_threads():
    try:
        from threadpoolctl import threadpool_info

        return max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001 - the count is informational
        return None


def cpu_baseline(value, unit, sample, numpy_oracle=False):
    """The reported host baseline: the C oracle (OpenMP over (sequence, head)
    units) or, for the softmax layer, the NumPy oracle (BLAS threads)."""
    import oracle

    return {"value": round(value, 3), "unit": unit,
            "cores": blas_threads() if numpy_oracle else oracle.max_threads(), "kind": "oracle",
            "sample": sample, "cpu": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
            "build": "NumPy fp64" if numpy_oracle else oracle_build()}


def prefill_oracle_baseline(q, k, v, slopes, cu, s0, tokens, what, min_seconds):
    """The fp64 oracle (recurrence over packed sequences, every head) on host
    copies of a bounded sample of a workload's inputs; tokens/s of that sample."""
    import oracle

    rate, reps, dt = oracle_rate(lambda: oracle.recurrence_packed(q, k, v, slopes, cu, s0=s0), tokens,
                                 min_seconds)
    return cpu_baseline(rate, "tokens/s", f"{what}, {reps} runs, {dt:.2f} s, fp64")


def host(x):
    return x.float().cpu().numpy()


# ---------------------------------------------------------------------------
# the M1-layer prefill (the benchmark line)

def run_m1_prefill(la, torch, steps, warmup, slope_scale=1.0):
    """lt_prefill on the M1 layer. slope_scale multiplies every head's slope
    (smaller slopes: longer memories, so more heads take the pre-pass instead
    of warm-up ranges); 1 is the benchmark line."""
    import numpy as np

    import workloads

    w = workloads.M1_LAYER
    shape = (w.batch, w.seqlen, w.heads, w.head_dim)
    q, k, v = workloads.qkv_device(w.seed, shape, "bf16")
    slopes = torch.from_numpy((workloads.slopes(w.heads) * np.float32(slope_scale)).astype(np.float32)).cuda()
    o = torch.empty(shape, device="cuda", dtype=torch.float32)
    st = torch.empty((w.batch, w.heads, D, D), device="cuda", dtype=torch.float32)
    stream = torch.cuda.current_stream()
    call = lambda: la.lt_prefill(q, k, v, slopes, w.block, o=o, state_out=st, stream=stream)
    ms, med, _, wall = time_calls(torch, call, steps, warmup, stream)
    assert bool(torch.isfinite(o[0, -1]).all()), "non-finite prefill output"
    tokens = w.batch * w.seqlen
    nbytes = prefill_bytes(tokens, w.heads)
    res = {"tokens_per_s": tokens * steps / wall, "ms_per_step": wall * 1e3 / steps, "kernel_ms_mean": ms,
           "kernel_ms_median": med,
           "roofline": hbm_roofline(nbytes, ms, "lt_prefill call: piece_state_kernel + "
                                    "head_kernel<float, false> + finish_kernel<float, false>",
                                    committed_traffic("m1_layer") if slope_scale == 1.0 else None)}
    return w, (q, k, v, slopes), res


def run_norm_gate(la, torch, steps, warmup):
    """lt_prefill_norm_gate on the M1 layer: bf16 q, k, v and gate, bf16 y, fp32
    final state; algorithmic bytes 3*256 + 256 + 256 = 1,280 B per token-head."""
    import workloads

    w = workloads.M1_LAYER
    shape = (w.batch, w.seqlen, w.heads, w.head_dim)
    q, k, v = workloads.qkv_device(w.seed, shape, "bf16")
    gate = workloads.gate_device(w.seed + 10, shape, "bf16")
    nw = torch.from_numpy(workloads.norm_weight_host(w.seed + 11, w.heads)).cuda()
    slopes = torch.from_numpy(workloads.slopes(w.heads)).cuda()
    y = torch.empty(shape, device="cuda", dtype=torch.bfloat16)
    st = torch.empty((w.batch, w.heads, D, D), device="cuda", dtype=torch.float32)
    stream = torch.cuda.current_stream()
    call = lambda: la.lt_prefill_norm_gate(q, k, v, slopes, gate, nw, workloads.NORM_EPS, w.block, y=y,
                                           state_out=st, stream=stream)
    ms, _, _, _ = time_calls(torch, call, steps, warmup, stream)
    assert bool(torch.isfinite(y[0, -1].float()).all()), "non-finite norm-gate output"
    tokens = w.batch * w.seqlen
    nbytes = tokens * w.heads * D * (3 * 2 + 2 + 2) + w.batch * w.heads * D * D * 4
    return {"workload": w.name + " + norm_gate", "gate_dtype": "bf16", "out_dtype": "bf16",
            "tokens_per_s": round(tokens / (ms / 1e3), 1), "kernel_ms_mean": round(ms, 5),
            "roofline": hbm_roofline(nbytes, ms, "lt_prefill_norm_gate call: piece_state_kernel + "
                                     "head_kernel<bf16, norm-gate> + finish_kernel<bf16, true>")}


def run_backward(la, torch, steps, warmup, batch, seqlen):
    """lt_prefill_backward on [batch, seqlen, 64, 128] bf16 with fp32 gradients and a
    final-state gradient. Algorithmic bytes: q, k, v, dO read once and dq, dk, dv
    written once (3 * 256 + 256 + 3 * 512 = 2,560 B per token-head) plus the states."""
    import workloads

    H = 64
    shape = (batch, seqlen, H, D)
    q, k, v = workloads.qkv_device(1002, shape, "bf16")
    do = workloads.gate_device(1020, shape, "bf16")
    slopes = torch.from_numpy(workloads.slopes(H)).cuda()
    ds = workloads.state_device(1021, (batch, H, D, D), std=0.1)
    dq, dk, dv = (torch.empty(shape, device="cuda", dtype=torch.float32) for _ in range(3))
    dsi = torch.empty((batch, H, D, D), device="cuda", dtype=torch.float32)
    stream = torch.cuda.current_stream()
    call = lambda: la.lt_prefill_backward(q, k, v, do, slopes, 256, None, ds, dq=dq, dk=dk, dv=dv,
                                          d_state_in=dsi, stream=stream)
    ms, _, _, _ = time_calls(torch, call, steps, warmup, stream)
    assert bool(torch.isfinite(dk[0, 0]).all()), "non-finite backward output"
    tokens = batch * seqlen
    nbytes = backward_bytes(batch, seqlen, H)
    name = f"backward_b{batch}_L{seqlen}"
    return {"workload": f"backward [{batch}, {seqlen}, {H}, {D}] bf16 -> fp32 grads",
            "tokens_per_s": round(tokens / (ms / 1e3), 1), "kernel_ms_mean": round(ms, 5),
            "roofline": hbm_roofline(nbytes, ms, "lt_prefill_backward call: dq forward pass + rev_piece_kernel "
                                     "+ bwd_kv_kernel + bwd_finish_kernel", committed_traffic(name))}


def backward_cpu_baseline(min_seconds):
    """The fp64 oracle backward on the first 4096 tokens of the M1-layer backward
    inputs, every head."""
    import numpy as np

    import oracle
    import workloads

    H, n = 64, 4096
    q, k, v = (host(x[:, :n]) for x in workloads.qkv_device(1002, (1, 32768, H, D), "bf16"))
    do = host(workloads.gate_device(1020, (1, 32768, H, D), "bf16")[:, :n])
    ds = host(workloads.state_device(1021, (1, H, D, D), std=0.1))
    sl = workloads.slopes(H)
    rate, reps, dt = oracle_rate(lambda: oracle.backward_batch(q, k, v, do, sl, ds=ds), n, min_seconds)
    return cpu_baseline(rate, "tokens/s", f"first {n} of 32768 tokens, all {H} heads, {reps} runs, {dt:.2f} s, fp64")


# ---------------------------------------------------------------------------
# decode

def decode_inputs(torch, nsteps, slots=0):
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
    state = workloads.state_device(w.seed, (max(B, slots), H, D, D), std=1.0)
    state.mul_(std.float().cuda().view(1, H, 1, 1))
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed + 1)
    qkv = (torch.randn((nsteps, 3, B, H, D), generator=g, device="cuda")
           .mul_(workloads.INPUT_SCALE).to(torch.bfloat16))
    return w, state, qkv


def run_decode(la, torch, nsteps, warmup=5, norm_gate=False, slots=0):
    """Batched decode steps (norm_gate: lt_decode_norm_gate with bf16 gate and
    bf16 y, the same algorithmic bytes as the plain step with fp32 o; slots > 0:
    lt_decode_slots with the batch's states scattered over a pool of that many
    slots, same algorithmic bytes plus 4 B of slot id per sequence)."""
    import numpy as np

    import workloads

    w, state, qkv = decode_inputs(torch, nsteps + warmup, slots)
    B, H = w.batch, w.heads
    slopes = torch.from_numpy(workloads.slopes(H)).cuda()
    stream = torch.cuda.current_stream()
    it = iter(range(nsteps + warmup))
    if slots:
        ids = torch.from_numpy(np.random.Generator(np.random.PCG64(w.seed + 4))
                               .permutation(slots)[:B].astype(np.int32)).cuda()
        o = torch.empty((B, H, D), device="cuda", dtype=torch.float32)

        def call():
            x = qkv[next(it)]
            la.lt_decode_slots(x[0], x[1], x[2], slopes, state, ids, o=o, stream=stream)
    elif norm_gate:
        gates = workloads.gate_device(w.seed + 2, (nsteps + warmup, B, H, D), "bf16")
        nw = torch.from_numpy(workloads.norm_weight_host(w.seed + 3, H)).cuda()
        o = torch.empty((B, H, D), device="cuda", dtype=torch.bfloat16)

        def call():
            i = next(it)
            x = qkv[i]
            la.lt_decode_norm_gate(x[0], x[1], x[2], slopes, state, gates[i], nw, workloads.NORM_EPS, y=o,
                                   stream=stream)
    else:
        o = torch.empty((B, H, D), device="cuda", dtype=torch.float32)

        def call():
            x = qkv[next(it)]
            la.lt_decode(x[0], x[1], x[2], slopes, state, o=o, stream=stream)
    _, med, ms, _ = time_calls(torch, call, nsteps, warmup, stream)
    assert bool(torch.isfinite(o).all()), "non-finite decode output"
    nbytes = decode_bytes(B, H) if not norm_gate else B * H * (2 * D * D * 4 + 4 * D * 2 + D * 2)
    nbytes += 4 * B if slots else 0
    kernel = ("decode_kernel<bf16, bf16, norm-gate>" if norm_gate else
              "decode_kernel<bf16, f32, slots>" if slots else "decode_kernel<bf16, f32>")
    return {
        "workload": w.name + (f" over a {slots}-slot state pool" if slots else ""),
        "batch": B, "heads": H, "head_dim": D, "steps": nsteps,
        "steps_per_s": round(1e3 / med, 1),
        "ms_per_step_median": round(med, 5),
        "ms_per_step_p10": round(float(np.percentile(ms, 10)), 5),
        "ms_per_step_p90": round(float(np.percentile(ms, 90)), 5),
        "roofline": hbm_roofline(nbytes, med, kernel,
                                 committed_traffic("decode") if not (slots or norm_gate) else None),
        "state": "Gaussian stand-in with the per-head scale of a 4096-token prefill state",
    }


def decode_cpu_baseline(min_seconds):
    """The fp64 oracle's decode step on 16 of the 256 sequences (all heads);
    reported as whole 256-sequence steps per second (the sample's rate / 16)."""
    import numpy as np

    import oracle
    import workloads

    B, H, n = 256, 64, 16
    g = np.random.Generator(np.random.PCG64(workloads.DECODE.seed))
    q, k, v = (workloads.round_bf16(g.standard_normal((n, H, D), dtype=np.float32) * np.float32(workloads.INPUT_SCALE))
               for _ in range(3))
    st = g.standard_normal((n, H, D, D)).astype(np.float32) * np.float32(0.05)
    sl = workloads.slopes(H)
    rate, reps, dt = oracle_rate(lambda: oracle.decode(q, k, v, sl, st), n, min_seconds, max_reps=2000)
    return cpu_baseline(rate / B, "steps/s",
                        f"{n} of the {B} sequences x {H} heads per step, {reps} steps, {dt:.2f} s, fp64; "
                        f"value = sequence-steps/s / {B} (extrapolated to whole steps)")


# ---------------------------------------------------------------------------
# the other workloads of the benchmark set

def run_tiny(la, torch, steps, warmup, cpu, min_seconds):
    import workloads

    w = workloads.TINY_F32
    shape = (w.batch, w.seqlen, w.heads, D)
    qh, kh, vh = workloads.qkv_host(w.seed, shape, "f32")
    q, k, v = (torch.from_numpy(x).cuda() for x in (qh, kh, vh))
    sl = workloads.slopes(w.heads)
    slopes = torch.from_numpy(sl).cuda()
    o = torch.empty(shape, device="cuda", dtype=torch.float32)
    st = torch.empty((w.batch, w.heads, D, D), device="cuda", dtype=torch.float32)
    stream = torch.cuda.current_stream()
    call = lambda: la.lt_prefill(q, k, v, slopes, w.block, o=o, state_out=st, stream=stream)
    ms, _, _, wall = time_calls(torch, call, steps, warmup, stream)
    tokens = w.batch * w.seqlen
    res = {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen, "heads": w.heads, "block": w.block,
           "dtype": "f32", "tokens_per_s": round(tokens * steps / wall, 1), "call_ms_mean": round(ms, 5),
           "roofline": hbm_roofline(prefill_bytes(tokens, w.heads, in_bytes=4), ms,
                                    "lt_prefill call: prefill_kernel<float, float> (fp32 MFMA)",
                                    committed_traffic("tiny_f32")),
           "note": "launch-bound: 8 (sequence, head) pairs x 4 value slices = 32 workgroups"}
    if cpu:
        res["cpu_baseline"] = prefill_oracle_baseline(
            qh.reshape(tokens, w.heads, D), kh.reshape(tokens, w.heads, D), vh.reshape(tokens, w.heads, D), sl,
            [0, tokens], None, tokens, f"the whole workload ({tokens} tokens x {w.heads} heads)", min_seconds)
    return res


def run_long_1m(la, torch, steps, warmup, cpu, min_seconds, sample=32768):
    import workloads

    w = workloads.LONG_1M
    shape = (w.batch, w.seqlen, w.heads, D)
    q, k, v = workloads.qkv_device(w.seed, shape, "bf16")
    sl = workloads.slopes(w.heads)
    slopes = torch.from_numpy(sl).cuda()
    o = torch.empty(shape, device="cuda", dtype=torch.float32)
    st = torch.empty((w.batch, w.heads, D, D), device="cuda", dtype=torch.float32)
    stream = torch.cuda.current_stream()
    call = lambda: la.lt_prefill(q, k, v, slopes, w.block, o=o, state_out=st, stream=stream)
    ms, _, _, wall = time_calls(torch, call, steps, warmup, stream)
    assert bool(torch.isfinite(o[0, -1]).all()), "non-finite 1M output"
    tokens = w.batch * w.seqlen
    res = {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen, "heads": w.heads, "block": w.block,
           "dtype": "bf16", "tokens_per_s": round(tokens * steps / wall, 1), "call_ms_mean": round(ms, 5),
           "roofline": hbm_roofline(prefill_bytes(tokens, w.heads), ms, "lt_prefill call",
                                    committed_traffic("long_1m"))}
    if cpu:
        hq, hk, hv = (host(x[0, :sample]) for x in (q, k, v))
        res["cpu_baseline"] = prefill_oracle_baseline(
            hq, hk, hv, sl, [0, sample], None, sample,
            f"first {sample} of {w.seqlen} tokens, all {w.heads} heads", min_seconds)
    del q, k, v, o
    torch.cuda.empty_cache()
    return res


def run_varlen(la, torch, steps, warmup, cpu, min_seconds):
    import workloads

    w = workloads.VARLEN
    H = w.heads
    lens = workloads.varlen_lengths(w.seed, w.batch, w.extra["min_len"], w.extra["max_len"])
    cu_h = workloads.cu_seqlens(lens)
    T, n = int(cu_h[-1]), len(lens)
    q, k, v = workloads.qkv_device(w.seed, (T, H, D), "bf16")
    cu = torch.from_numpy(cu_h).cuda()
    s0 = workloads.state_device(w.seed + 1, (n, H, D, D), std=0.1)
    sl = workloads.slopes(H)
    slopes = torch.from_numpy(sl).cuda()
    o = torch.empty((T, H, D), device="cuda", dtype=torch.float32)
    st = torch.empty_like(s0)
    stream = torch.cuda.current_stream()
    mx = int(lens.max())
    call = lambda: la.lt_prefill_varlen(q, k, v, cu, slopes, w.block, s0, max_seqlen=mx, o=o, state_out=st,
                                        stream=stream)
    ms, _, _, wall = time_calls(torch, call, steps, warmup, stream)
    res = {"workload": w.name, "num_seqs": n, "total_tokens": T, "min_len": int(lens.min()), "max_len": mx,
           "heads": H, "block": w.block, "dtype": "bf16", "tokens_per_s": round(T * steps / wall, 1),
           "call_ms_mean": round(ms, 5),
           "roofline": hbm_roofline(prefill_bytes(T, H, states_out=n, states_in=n), ms, "lt_prefill_varlen call",
                                    committed_traffic("varlen"))}
    if cpu:
        # the first two sequences in full, with their carried-in states
        a2 = int(cu_h[2])
        hq, hk, hv = (host(x[:a2]) for x in (q, k, v))
        res["cpu_baseline"] = prefill_oracle_baseline(
            hq, hk, hv, sl, cu_h[:3], host(s0[:2]), a2,
            f"sequences 0 and 1 ({int(lens[0])} + {int(lens[1])} tokens) with their carried states, "
            f"all {H} heads", min_seconds)
    del q, k, v, o
    torch.cuda.empty_cache()
    return res


def run_varlen_2x(la, torch, steps, warmup, cpu, min_seconds, sample=16384, compare=True):
    """A packed batch of 2 x 131072 tokens with carried states, beside lt_prefill
    on the same [2, 131072] batch (the packed call splits its long sequences the
    same way)."""
    import workloads

    L, H, n = 131072, 64, 2
    q, k, v = workloads.qkv_device(6301, (n, L, H, D), "bf16")
    s0 = workloads.state_device(6302, (n, H, D, D), std=0.1)
    sl = workloads.slopes(H)
    slopes = torch.from_numpy(sl).cuda()
    o = torch.empty((n, L, H, D), device="cuda", dtype=torch.float32)
    st = torch.empty_like(s0)
    cu = torch.tensor([0, L, 2 * L], dtype=torch.int32, device="cuda")
    flat = lambda x: x.view(n * L, H, D)
    stream = torch.cuda.current_stream()
    vcall = lambda: la.lt_prefill_varlen(flat(q), flat(k), flat(v), cu, slopes, 256, s0, max_seqlen=L,
                                         o=flat(o), state_out=st, stream=stream)
    fcall = lambda: la.lt_prefill(q, k, v, slopes, 256, s0, o=o, state_out=st, stream=stream)
    ms, _, _, wall = time_calls(torch, vcall, steps, warmup, stream)
    # the same-shape lt_prefill calls are left out of a counter run (compare=False),
    # so that its dispatches are the packed calls alone
    fms = time_calls(torch, fcall, steps, warmup, stream)[0] if compare else None
    tokens = n * L
    nbytes = prefill_bytes(tokens, H, states_out=n, states_in=n)
    res = {"workload": "varlen_2x131072_carried_state_prefill", "num_seqs": n, "total_tokens": tokens,
           "heads": H, "block": 256, "dtype": "bf16", "tokens_per_s": round(tokens * steps / wall, 1),
           "call_ms_mean": round(ms, 5),
           "lt_prefill_same_shape_ms_mean": round(fms, 5) if compare else None,
           "rate_vs_lt_prefill": round(fms / ms, 4) if compare else None,
           "roofline": hbm_roofline(nbytes, ms, "lt_prefill_varlen call", committed_traffic("varlen_2x131072"))}
    if cpu:
        hq, hk, hv = (host(torch.cat([x[0, :sample], x[1, :sample]])) for x in (q, k, v))
        res["cpu_baseline"] = prefill_oracle_baseline(
            hq, hk, hv, sl, [0, sample, 2 * sample], host(s0), 2 * sample,
            f"first {sample} tokens of each sequence with their carried states, all {H} heads", min_seconds)
    del q, k, v, o
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# the softmax layer

def run_softmax(la, torch, steps, warmup, decode_steps):
    """The hybrid's softmax attention layer (64 query heads, 8 K/V heads of 128,
    RoPE on 64 dims): causal prefill of 32768 tokens (bf16 in, bf16 out) against
    the bf16 MFMA peak (algorithmic FLOPs 2 * Hq * L^2 * d, the causal half of
    the two products), and a decode step of 16 sequences over 32768 cached tokens
    each against HBM (algorithmic bytes: the K and V cache rows read, 0..n)."""
    import workloads

    wl = workloads.SOFTMAX_PREFILL
    B, L, Hq, Hkv = wl.batch, wl.seqlen, wl.heads, wl.extra["kv_heads"]
    R, base = wl.extra["rope_dims"], wl.extra["rope_base"]
    q, k, v = workloads.softmax_qkv_device(wl.seed, B, L, Hq, Hkv)
    o = torch.empty((B, L, Hq, D), device="cuda", dtype=torch.bfloat16)
    kr = torch.empty_like(k)
    stream = torch.cuda.current_stream()
    call = lambda: la.lt_softmax_prefill(q, k, v, rope_dims=R, rope_base=base, o=o, k_rope=kr, stream=stream)
    ms, _, _, _ = time_calls(torch, call, steps, warmup, stream)
    assert bool(torch.isfinite(o[0, -1]).all()), "non-finite softmax output"
    flops = 2.0 * B * Hq * L * L * D
    tfs = flops / (ms / 1e3) / 1e12
    pre = {"workload": f"{wl.name}: [{B}, {L}] x {Hq} query / {Hkv} K/V heads x {D}, rope {R}",
           "tokens_per_s": round(B * L / (ms / 1e3), 1), "call_ms_mean": round(ms, 4),
           "roofline": {"bound": "mfma", "achieved": round(tfs, 1), "peak": MFMA_BF16_PEAK_TFS,
                        "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4), "flops_per_launch": flops,
                        "kernel": "lt_softmax_prefill call: rope_rows_kernel + fa_prefill_kernel<bf16>"}}
    del q, k, v, o, kr
    wd = workloads.SOFTMAX_DECODE
    Bd, ctx = wd.batch, wd.extra["context"]
    cap = ctx + 1024
    g = torch.Generator(device="cuda")
    g.manual_seed(wd.seed)
    rnd = lambda *sh: torch.randn(sh, generator=g, device="cuda").to(torch.bfloat16)
    dq, kn, vn = rnd(Bd, Hq, D), rnd(Bd, Hkv, D), rnd(Bd, Hkv, D)
    kc, vc = rnd(Bd, cap, Hkv, D), rnd(Bd, cap, Hkv, D)
    lens = torch.full((Bd,), ctx, dtype=torch.int32, device="cuda")
    do = torch.empty((Bd, Hq, D), device="cuda", dtype=torch.bfloat16)
    ws = torch.empty(max(la.lt_softmax_decode_workspace_bytes(Bd, cap, Hq, Hkv), 1), dtype=torch.uint8,
                     device="cuda")
    dcall = lambda: la.lt_softmax_decode(dq, kn, vn, kc, vc, lens, rope_dims=R, rope_base=base, o=do,
                                         workspace=ws, stream=stream)
    dms, dmed, _, _ = time_calls(torch, dcall, decode_steps, 5, stream)
    nbytes = Bd * (ctx + 1) * Hkv * D * 2 * 2
    dec = {"workload": f"{wd.name}: {Bd} sequences x {ctx} cached tokens, {Hq} / {Hkv} heads, bf16 cache",
           "ms_per_step_mean": round(dms, 5), "ms_per_step_median": round(dmed, 5),
           "roofline": hbm_roofline(nbytes, dms, "lt_softmax_decode call: rope_append + fd_kernel + fd_combine")}
    del kc, vc
    torch.cuda.empty_cache()
    return {"prefill": pre, "decode": dec}


def run_softmax_cpu_baseline(min_seconds=5.0):
    """The fp64 softmax oracle on the host, beside the GPU softmax rows: query
    rows of the same 32768-token layer spread evenly over [0, L) (so their mean
    cost is that of an average row), and decode steps of single sequences over
    the same 32768-token context. Reported baseline, not a target."""
    import numpy as np

    import oracle
    import workloads

    wl = workloads.SOFTMAX_PREFILL
    B, L, Hq, Hkv = wl.batch, wl.seqlen, wl.heads, wl.extra["kv_heads"]
    R, base = wl.extra["rope_dims"], wl.extra["rope_base"]
    q, k, v = workloads.softmax_qkv_device(wl.seed, B, L, Hq, Hkv)
    hq, hk, hv = (host(x) for x in (q, k, v))
    del q, k, v
    rows_done, dt, passes = 0, 0.0, 0
    while dt < min_seconds and passes < 64:
        rows = np.arange((509 * passes) % 4096, L, 4096)[:8]  # 8 rows 4096 apart, offset per pass
        t0 = time.perf_counter()
        oracle.softmax_attention_rows(hq, hk, hv, rows, rope_dims=R, base=base)
        dt += time.perf_counter() - t0
        rows_done += len(rows)
        passes += 1
    pre = cpu_baseline(rows_done / dt, "tokens/s",
                       f"{rows_done} query rows x {Hq} heads spread over [0, {L}), {dt:.2f} s, fp64",
                       numpy_oracle=True)
    wd = workloads.SOFTMAX_DECODE
    ctx = wd.extra["context"]
    g = np.random.Generator(np.random.PCG64(wd.seed))
    kc = g.standard_normal((1, ctx + 1, Hkv, D))
    vc = g.standard_normal((1, ctx + 1, Hkv, D))
    qd, kn, vn = g.standard_normal((1, Hq, D)), g.standard_normal((1, Hkv, D)), g.standard_normal((1, Hkv, D))
    steps, dt = 0, 0.0
    while dt < min_seconds and steps < 200:
        t0 = time.perf_counter()
        oracle.softmax_decode(qd, kn, vn, kc, vc, np.array([ctx]), rope_dims=R, base=base)
        dt += time.perf_counter() - t0
        steps += 1
    dec = cpu_baseline(steps / dt, "sequence-steps/s",
                       f"{steps} decode steps of one sequence over {ctx} cached tokens, {Hq} / {Hkv} heads, "
                       f"{dt:.2f} s, fp64 (the GPU step serves {wd.batch} sequences)", numpy_oracle=True)
    return {"prefill": pre, "decode": dec}


# ---------------------------------------------------------------------------
# counter traffic

def copy_calibration(torch, nbytes):
    """A plain copy kernel of nbytes (reads nbytes, writes nbytes): torch's
    elementwise kernel for dst = src * 1 (a same-dtype copy_ could go to the
    DMA engine, which the shader counters do not see)."""
    src = torch.ones(nbytes // 4, device="cuda", dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes}))


def traffic_from(copy_dir, fetch_dir, write_dir, copy_bytes, workload, calls):
    """Per-call HBM traffic of `bench.py --only WORKLOAD` from rocprofv3 runs.

    copy_dir holds FETCH_SIZE (copy_dir/fetch) and WRITE_SIZE (copy_dir/write)
    of the calibration copy; fetch_dir and write_dir hold FETCH_SIZE and
    WRITE_SIZE of a `--only WORKLOAD` run of `calls` calls (warm-ups included).
    Each counter is scaled by (bytes the copy moved) / (what the counter read
    for the copy); the library's kernels' totals over the run are divided by
    `calls`. Writes the entry into profiles/traffic_counters.json.
    """
    import csv
    import glob

    def per_kernel(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    cf = per_kernel(os.path.join(copy_dir, "fetch"), "FETCH_SIZE")
    cw = per_kernel(os.path.join(copy_dir, "write"), "WRITE_SIZE")
    ck = [k for k in cf if "copy" in k.lower() or "elementwise" in k.lower()]
    copy_fetch_kib = max(max(cf[k]) for k in ck)
    copy_write_kib = max(max(cw[k]) for k in cw if k in ck)
    f_scale = copy_bytes / (copy_fetch_kib * 1024)
    w_scale = copy_bytes / (copy_write_kib * 1024)
    kf = per_kernel(fetch_dir, "FETCH_SIZE")
    kw = per_kernel(write_dir, "WRITE_SIZE")
    import re

    def short(k):  # "void lt::(anonymous namespace)::head_kernel<float, false>(...)" -> head_kernel<float, false>
        m = re.search(r"lt::(?:\(anonymous namespace\)::)?(\w+(?:<[^()]*>)?)\(", k)
        return m.group(1) if m else k

    kernels = sorted(k for k in kf if "lt::" in k)
    per = {}
    for k in kernels:
        per[short(k)] = {"calls": len(kf[k]), "fetch_bytes": round(sum(kf[k]) * 1024 * f_scale / calls),
                         "write_bytes": round(sum(kw.get(k, [])) * 1024 * w_scale / calls)}
    fetch = sum(p["fetch_bytes"] for p in per.values())
    write = sum(p["write_bytes"] for p in per.values())
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    table[workload] = {"sources_hash": sources_hash(workload), "calls": calls, "fetch_scale": f_scale,
                       "write_scale": w_scale, "fetch_bytes_per_call": fetch, "write_bytes_per_call": write,
                       "traffic_bytes_per_call": fetch + write, "per_kernel_per_call": per}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    print(json.dumps({workload: table[workload]}))


# ---------------------------------------------------------------------------

def run_only(la, torch, name, steps, warmup):
    """One workload alone (for profiler passes); prints its JSON."""
    if name == "m1_layer":
        _, _, r = run_m1_prefill(la, torch, steps, warmup)
    elif name == "decode":
        r = run_decode(la, torch, steps, warmup)
    elif name.startswith("backward"):
        b, L = (1, 32768) if name == "backward_b1_L32768" else (4, 8192)
        r = run_backward(la, torch, steps, warmup, b, L)
    elif name == "tiny_f32":
        r = run_tiny(la, torch, steps, warmup, False, 0)
    elif name == "long_1m":
        r = run_long_1m(la, torch, steps, warmup, False, 0)
    elif name == "varlen":
        r = run_varlen(la, torch, steps, warmup, False, 0)
    elif name == "varlen_2x131072":
        r = run_varlen_2x(la, torch, steps, warmup, False, 0, compare=False)
    else:
        raise SystemExit(f"unknown workload {name}")
    print(json.dumps({"only": name, "steps": steps, "warmup": warmup, "result": r}), flush=True)


ONLY = ("m1_layer", "decode", "backward_b1_L32768", "backward_b4_L8192", "tiny_f32", "long_1m", "varlen",
        "varlen_2x131072")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # Untimed calls before each timed workload (after settle_gpu; without it a
    # burst of back-to-back calls after idle starts slow for about 30 calls).
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--cpu-tokens", type=int, default=32768)
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-settle", action="store_true",
                    help="time from an idle GPU (no settle_gpu before each workload)")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-norm-gate", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-softmax", action="store_true")
    ap.add_argument("--no-slopes-scaled", action="store_true",
                    help="skip the prefill runs with scaled-down slopes")
    ap.add_argument("--norm-gate-decode-steps", type=int, default=200)
    ap.add_argument("--only", choices=ONLY)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--traffic-from", nargs=3, metavar=("COPY_DIR", "FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--traffic-workload", choices=ONLY, default="m1_layer")
    ap.add_argument("--calls", type=int, default=0, help="calls of the profiled --only run (warm-ups included)")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    args = ap.parse_args()
    _SETTLE["on"] = not args.no_settle
    if args.traffic_from:
        traffic_from(*args.traffic_from, args.copy_bytes, args.traffic_workload, args.calls)
        return

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

    # the library's GPU code is loaded here, not inside the first timed
    # workload's first calls (a few milliseconds of host work that leave the
    # GPU idle after settle_gpu)
    la.lt_init()
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
        return
    if args.only:
        log(f"[bench] only {args.only}: {args.warmup} + {args.steps} calls")
        run_only(la, torch, args.only, args.steps, args.warmup)
        return

    cpu_s = args.cpu_seconds
    log("[bench] prefill m1_layer L=32768 H=64 d=128 block=256")
    w, dev_inputs, pre = run_m1_prefill(la, torch, args.steps, args.warmup)
    log(f"[bench] prefill {pre['kernel_ms_mean']:.3f} ms/call")
    scaled = {}
    for f in (() if args.no_slopes_scaled else (0.1, 1e-5)):
        _, _, r = run_m1_prefill(la, torch, 10, 20, slope_scale=f)
        scaled[f"x{f:g}"] = {"kernel_ms_mean": round(r["kernel_ms_mean"], 5),
                             "tokens_per_s": round(1e3 * w.batch * w.seqlen / r["kernel_ms_mean"], 1),
                             "roofline_frac": r["roofline"]["frac"]}
        log(f"[bench] prefill, slopes x{f:g}: {r['kernel_ms_mean']:.3f} ms/call")
    cpu = None
    if not args.no_cpu:
        log(f"[bench] cpu oracle on {args.cpu_tokens} tokens")
        tokens = min(args.cpu_tokens, w.seqlen)
        q, k, v, slopes = dev_inputs
        hq, hk, hv = (host(x[0, :tokens]) for x in (q, k, v))
        cpu = prefill_oracle_baseline(hq, hk, hv, slopes.cpu().numpy(), [0, tokens], None, tokens,
                                      f"first {tokens} of {w.seqlen} tokens, all {w.heads} heads",
                                      max(cpu_s, 10.0))
    del dev_inputs
    torch.cuda.empty_cache()
    configs = None
    if not args.no_configs:
        configs = {}
        log("[bench] tiny fp32 prefill")
        configs["tiny_f32"] = run_tiny(la, torch, 20, 3, not args.no_cpu, cpu_s / 2)
        log(f"[bench] 1M-token prefill")
        configs["long_1m"] = run_long_1m(la, torch, 5, 2, not args.no_cpu, cpu_s)
        log(f"[bench] 1M {configs['long_1m']['call_ms_mean']:.3f} ms/call")
        log("[bench] varlen prefill, 16 sequences with carried states")
        configs["varlen"] = run_varlen(la, torch, 10, 2, not args.no_cpu, cpu_s)
        log(f"[bench] varlen {configs['varlen']['call_ms_mean']:.3f} ms/call")
        log("[bench] varlen prefill, 2 x 131072 tokens")
        configs["varlen_2x131072"] = run_varlen_2x(la, torch, 10, 4, not args.no_cpu, cpu_s / 2)
        log(f"[bench] varlen 2x131072 {configs['varlen_2x131072']['call_ms_mean']:.3f} ms/call "
            f"(lt_prefill {configs['varlen_2x131072']['lt_prefill_same_shape_ms_mean']:.3f})")
    dec = None
    if not args.no_decode:
        log(f"[bench] decode batch=256 H=64, {args.decode_steps} steps")
        dec = run_decode(la, torch, args.decode_steps)
        log(f"[bench] decode {dec['ms_per_step_median']:.4f} ms/step")
        dec["slots"] = run_decode(la, torch, args.norm_gate_decode_steps, slots=512)
        log(f"[bench] decode over 512 slots {dec['slots']['ms_per_step_median']:.4f} ms/step")
        if not args.no_cpu:
            dec["cpu_baseline"] = decode_cpu_baseline(cpu_s / 2)
        torch.cuda.empty_cache()
    ng = None
    if not args.no_norm_gate:
        log("[bench] prefill + norm_gate m1_layer (bf16 gate, bf16 y)")
        ng = {"prefill": run_norm_gate(la, torch, args.steps, args.warmup)}
        log(f"[bench] prefill + norm_gate {ng['prefill']['kernel_ms_mean']:.3f} ms/call")
        if not args.no_decode:
            ng["decode"] = run_decode(la, torch, args.norm_gate_decode_steps, norm_gate=True)
            log(f"[bench] decode + norm_gate {ng['decode']['ms_per_step_median']:.4f} ms/step")
        torch.cuda.empty_cache()
    bwd = None
    if not args.no_backward:
        bwd = {}
        for b_, l_ in ((1, 32768), (4, 8192)):
            log(f"[bench] backward batch={b_} L={l_} H=64")
            # 30 untimed calls (about 40 ms) carry the GPU past the slower stretch
            # that follows the start of a burst of back-to-back calls (as for the
            # M1 prefill line)
            bwd[f"b{b_}_L{l_}"] = run_backward(la, torch, 20, 30, b_, l_)
            log(f"[bench] backward {bwd[f'b{b_}_L{l_}']['kernel_ms_mean']:.3f} ms/call")
        if not args.no_cpu:
            bwd["cpu_baseline"] = backward_cpu_baseline(cpu_s / 2)
        torch.cuda.empty_cache()
    smx = None
    if not args.no_softmax:
        log("[bench] softmax layer: prefill L=32768 64/8 heads, decode 16 x 32768")
        smx = run_softmax(la, torch, 5, 1, 100)
        log(f"[bench] softmax prefill {smx['prefill']['call_ms_mean']:.3f} ms, decode "
            f"{smx['decode']['ms_per_step_median'] * 1e3:.1f} us")
        if not args.no_cpu:
            log("[bench] softmax oracle on the host")
            sb = run_softmax_cpu_baseline(cpu_s / 2)
            smx["prefill"]["cpu_baseline"], smx["decode"]["cpu_baseline"] = sb["prefill"], sb["decode"]

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
        "kernel_ms_median": round(pre["kernel_ms_median"], 5),
        # before each timed workload: 40 bf16 8192^3 matrix products (settle_gpu)
        # bring the GPU out of its post-idle state; null with --no-settle
        "gpu_settle": "40 x bf16 8192^3 matmul before warm-up" if _SETTLE["on"] else None,
        # the same call with every slope scaled down (x0.1: 15 of the 64 heads
        # take the pre-pass; x1e-5: all of them)
        "prefill_slopes_scaled": scaled,
        "configs": configs,
        "decode": dec,
        "norm_gate": ng,
        "backward": bwd,
        "softmax": smx,
        "cpu_baseline": cpu,
        "library_build_id": la.lib.lt_build_id().decode(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
