#!/usr/bin/env python3
"""Lightning Attention benchmark on one MI355X.

One step = one ``lt_prefill`` over the M1 Lightning-layer workload: batch 1,
L = 32768 tokens, 64 heads x 128, block 256, bf16 Q/K/V, fp32 O and fp32 final
state (the block form of MiniMax Signal Lab · M1, §03, on the layer shape of
§02/§04). Inputs are seeded synthetic tensors already resident in HBM.

Prints ONE JSON line. Besides the standard fields (metric, value, unit, steps, config ...) it carries:
  roofline      prefill kernel: algorithmic bytes per launch / mean launch
                duration (HIP events on the launch stream) against 8 TB/s HBM;
                ``traffic`` from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
                summary when it was taken on the current kernel source;
  decode        the batched decode step (256 sequences x 64 heads, 1 GiB fp32
                state updated in place), per-step HIP-event times over the run,
                state-stream GB/s against 8 TB/s;
  norm_gate     the same prefill and decode with the normalisation and gate
                fused into the epilogue (bf16 gate, bf16 y);
  backward      lt_prefill_backward (dq, dk, dv, dS0) on the M1 layer and on a
                4 x 8192-token batch of the same heads;
  softmax       the hybrid's softmax attention layer (§02: 64 query / 8 K/V
                heads, partial RoPE): causal prefill of 32768 tokens against the
                bf16 MFMA peak, and a 16 x 32768-token KV-cache decode step
                against HBM;
  cpu_baseline  the fp64 oracle on the host cores, timed on the same prefill
                workload (reported baseline, not a target).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps N]
                       [--no-cpu] [--no-decode] [--no-norm-gate] [--no-backward]
                       [--no-softmax]
       python bench.py --workload long_1m|varlen|tiny_f32   (one extra workload)
       python bench.py --copy-calibration BYTES            (plain device copy, for
                                                            rocprofv3 counter scaling)
       python bench.py --traffic-from COPY_DIR FETCH_DIR WRITE_DIR
                       (turn three rocprofv3 --pmc CSV runs into the per-launch
                        HBM traffic summary under profiles/)
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
# the prefill kernels and their launch plan: the committed traffic summary is
# valid while these sources are unchanged
PREFILL_SRCS = [os.path.join(ROOT, "linear_attention_amd", "csrc", f)
                for f in ("prefill_heads.hip", "tiles.h", "lightning_api.cpp")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def prefill_bytes(tokens, heads, in_bytes=2, out_bytes=4, states_out=1, states_in=0):
    """Algorithmic HBM bytes of one prefill: read q, k, v once, write o once,
    write (and read) the d x d fp32 states once."""
    return tokens * heads * D * (3 * in_bytes + out_bytes) + (states_out + states_in) * heads * D * D * 4


def decode_bytes(batch, heads, in_bytes=2, out_bytes=4):
    """Algorithmic HBM bytes of one decode step: state read + write, q, k, v, o."""
    return batch * heads * (2 * D * D * 4 + 3 * D * in_bytes + D * out_bytes)


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic(bytes_alg):
    """Per-launch HBM traffic from the committed rocprofv3 counter summary, if it
    was taken on the current prefill kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != source_sha(PREFILL_SRCS):
        return None
    return t.get("traffic_bytes_per_launch")


def run_prefill(la, torch, steps, warmup, slope_scale=1.0):
    """lt_prefill on the M1 layer. slope_scale multiplies every head's slope
    (smaller slopes: longer memories, so more heads take the pre-pass instead
    of local-start segments); 1 is the benchmark line."""
    import numpy as np

    import workloads

    w = workloads.M1_LAYER
    shape = (w.batch, w.seqlen, w.heads, w.head_dim)
    q, k, v = workloads.qkv_device(w.seed, shape, "bf16")
    slopes = torch.from_numpy((workloads.slopes(w.heads) * np.float32(slope_scale)).astype(np.float32)).cuda()
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
                     "kernel": "lt_prefill call: piece_state_kernel + combine_kernel + head_kernel<float> "
                               "+ fix_kernel<float, false>"},
    }


def run_prefill_norm_gate(la, torch, steps, warmup):
    """lt_prefill_norm_gate on the M1 layer: bf16 q, k, v and gate, bf16 y, fp32
    final state; algorithmic bytes 3*256 + 256 + 256 = 1,280 B per token-head."""
    import numpy as np

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

    def call():
        la.lt_prefill_norm_gate(q, k, v, slopes, gate, nw, workloads.NORM_EPS, w.block, y=y,
                                state_out=st, stream=stream)
    for _ in range(warmup):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    assert bool(torch.isfinite(y[0, -1].float()).all()), "non-finite norm-gate output"
    tokens = w.batch * w.seqlen
    nbytes = tokens * w.heads * D * (3 * 2 + 2 + 2) + w.batch * w.heads * D * D * 4
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"workload": w.name + " + norm_gate", "gate_dtype": "bf16", "out_dtype": "bf16",
            "tokens_per_s": round(tokens / (ms / 1e3), 1), "kernel_ms_mean": round(ms, 5),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "bytes_per_launch": nbytes,
                         "kernel": "lt_prefill_norm_gate call: piece_state_kernel + combine_kernel "
                                   "+ head_kernel<bf16, norm-gate> + fix_kernel<bf16, true>"}}


def run_backward(la, torch, steps, warmup, batch, seqlen):
    """lt_prefill_backward on [batch, seqlen, 64, 128] bf16 with fp32 gradients and a
    final-state gradient. Algorithmic bytes: q, k, v, dO read once and dq, dk, dv
    written once (3 * 256 + 256 + 3 * 512 = 2,560 B per token-head) plus the states."""
    import numpy as np

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

    def call():
        la.lt_prefill_backward(q, k, v, do, slopes, 256, None, ds, dq=dq, dk=dk, dv=dv,
                               d_state_in=dsi, stream=stream)
    for _ in range(warmup):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    assert bool(torch.isfinite(dk[0, 0]).all()), "non-finite backward output"
    tokens = batch * seqlen
    nbytes = tokens * H * D * (4 * 2 + 3 * 4) + 2 * batch * H * D * D * 4
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"workload": f"backward [{batch}, {seqlen}, {H}, {D}] bf16 -> fp32 grads",
            "tokens_per_s": round(tokens / (ms / 1e3), 1), "kernel_ms_mean": round(ms, 5),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "bytes_per_launch": nbytes,
                         "kernel": "lt_prefill_backward call: dq forward pass + rev_piece_kernel "
                                   "+ combine_kernel + bwd_kv_kernel + rev_fix_kernel"}}


MFMA_BF16_PEAK_TFS = 2500.0


def _event_times(torch, call, steps, warmup, stream):
    import numpy as np

    for _ in range(warmup):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) for a, b in ev]
    return float(np.mean(t)), float(np.median(t))


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
    ms, _ = _event_times(torch, call, steps, warmup, stream)
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
    dms, dmed = _event_times(torch, dcall, decode_steps, 5, stream)
    nbytes = Bd * (ctx + 1) * Hkv * D * 2 * 2
    gbs = nbytes / (dms / 1e3) / 1e9
    dec = {"workload": f"{wd.name}: {Bd} sequences x {ctx} cached tokens, {Hq} / {Hkv} heads, bf16 cache",
           "ms_per_step_mean": round(dms, 5), "ms_per_step_median": round(dmed, 5),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": nbytes,
                        "kernel": "lt_softmax_decode call: rope_append + fd_kernel + fd_combine"}}
    return {"prefill": pre, "decode": dec}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info

        return max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001 - the count is informational
        return None


def run_softmax_cpu_baseline(la, torch, min_seconds=5.0):
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
    hq, hk, hv = (x.float().cpu().numpy() for x in (q, k, v))
    del q, k, v
    rows_done, dt, passes = 0, 0.0, 0
    while dt < min_seconds and passes < 64:
        rows = np.arange((509 * passes) % 4096, L, 4096)[:8]  # 8 rows 4096 apart, offset per pass
        t0 = time.perf_counter()
        oracle.softmax_attention_rows(hq, hk, hv, rows, rope_dims=R, base=base)
        dt += time.perf_counter() - t0
        rows_done += len(rows)
        passes += 1
    pre = {"value": round(rows_done / dt, 2), "unit": "tokens/s", "cores": _blas_threads(), "kind": "oracle",
           "sample": f"{rows_done} query rows x {Hq} heads spread over [0, {L}), {dt:.2f} s, fp64"}
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
    dec = {"value": round(steps / dt, 3), "unit": "sequence-steps/s", "cores": _blas_threads(), "kind": "oracle",
           "sample": f"{steps} decode steps of one sequence over {ctx} cached tokens, {Hq} / {Hkv} heads, "
                     f"{dt:.2f} s, fp64 (the GPU step serves {wd.batch} sequences)"}
    return {"prefill": pre, "decode": dec}


def run_decode(la, torch, nsteps, warmup=5, norm_gate=False, slots=0):
    """Batched decode steps (norm_gate: lt_decode_norm_gate with bf16 gate and
    bf16 y, the same algorithmic bytes as the plain step with fp32 o; slots > 0:
    lt_decode_slots with the batch's states scattered over a pool of that many
    slots, same algorithmic bytes plus 4 B of slot id per sequence)."""
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
    state = workloads.state_device(w.seed, (max(B, slots), H, D, D), std=1.0)
    state.mul_(std.float().cuda().view(1, H, 1, 1))
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed + 1)
    qkv = (torch.randn((nsteps + warmup, 3, B, H, D), generator=g, device="cuda")
           .mul_(workloads.INPUT_SCALE).to(torch.bfloat16))
    slopes = torch.from_numpy(workloads.slopes(H)).cuda()
    stream = torch.cuda.current_stream()
    if slots:
        import numpy as _np
        ids = torch.from_numpy(_np.random.Generator(_np.random.PCG64(w.seed + 4))
                               .permutation(slots)[:B].astype(_np.int32)).cuda()
        o = torch.empty((B, H, D), device="cuda", dtype=torch.float32)

        def step(i):
            x = qkv[i]
            la.lt_decode_slots(x[0], x[1], x[2], slopes, state, ids, o=o, stream=stream)
    elif norm_gate:
        gates = workloads.gate_device(w.seed + 2, (nsteps + warmup, B, H, D), "bf16")
        nw = torch.from_numpy(workloads.norm_weight_host(w.seed + 3, H)).cuda()
        o = torch.empty((B, H, D), device="cuda", dtype=torch.bfloat16)

        def step(i):
            x = qkv[i]
            la.lt_decode_norm_gate(x[0], x[1], x[2], slopes, state, gates[i], nw,
                                   workloads.NORM_EPS, y=o, stream=stream)
    else:
        o = torch.empty((B, H, D), device="cuda", dtype=torch.float32)

        def step(i):
            x = qkv[i]
            la.lt_decode(x[0], x[1], x[2], slopes, state, o=o, stream=stream)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(nsteps)]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        step(warmup + i)
        b.record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    assert bool(torch.isfinite(o).all()), "non-finite decode output"
    med = float(np.median(ms))
    nbytes = decode_bytes(B, H) if not norm_gate else B * H * (2 * D * D * 4 + 4 * D * 2 + D * 2)
    nbytes += 4 * B if slots else 0
    gbs = nbytes / (med / 1e3) / 1e9
    return {
        "workload": w.name + (f" over a {slots}-slot state pool" if slots else ""),
        "batch": B, "heads": H, "head_dim": D, "steps": nsteps,
        "steps_per_s": round(1e3 / med, 1),
        "ms_per_step_median": round(med, 5),
        "ms_per_step_p10": round(float(np.percentile(ms, 10)), 5),
        "ms_per_step_p90": round(float(np.percentile(ms, 90)), 5),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": nbytes,
                     "kernel": ("decode_kernel<bf16, bf16, norm-gate>" if norm_gate else
                                "decode_kernel<bf16, f32, slots>" if slots else "decode_kernel<bf16, f32>")},
        "state": "Gaussian stand-in with the per-head scale of a 4096-token prefill state",
    }


def run_other(la, torch, name, steps, warmup):
    """Times one of the other workloads (prefill) and returns its JSON line."""
    import numpy as np

    import workloads

    w = {"long_1m": workloads.LONG_1M, "varlen": workloads.VARLEN,
         "tiny_f32": workloads.TINY_F32}[name]
    H = w.heads
    slopes = torch.from_numpy(workloads.slopes(H)).cuda()
    stream = torch.cuda.current_stream()
    if name == "varlen":
        lens = workloads.varlen_lengths(w.seed, w.batch, w.extra["min_len"], w.extra["max_len"])
        cu_h = workloads.cu_seqlens(lens)
        T = int(cu_h[-1])
        q, k, v = workloads.qkv_device(w.seed, (T, H, D), "bf16")
        cu = torch.from_numpy(cu_h).cuda()
        s0 = workloads.state_device(w.seed + 1, (len(lens), H, D, D), std=0.1)
        o = torch.empty((T, H, D), device="cuda", dtype=torch.float32)
        st = torch.empty_like(s0)
        call = lambda: la.lt_prefill_varlen(q, k, v, cu, slopes, w.block, s0, o=o, state_out=st,
                                            stream=stream)
        tokens, nbytes = T, prefill_bytes(T, H, states_out=len(lens), states_in=len(lens))
        cfg = {"num_seqs": len(lens), "total_tokens": T, "min_len": int(lens.min()),
               "max_len": int(lens.max())}
    else:
        dt = "f32" if name == "tiny_f32" else "bf16"
        shape = (w.batch, w.seqlen, H, D)
        if dt == "f32":
            q, k, v = (torch.from_numpy(x).cuda() for x in workloads.qkv_host(w.seed, shape, "f32"))
        else:
            q, k, v = workloads.qkv_device(w.seed, shape, "bf16")
        o = torch.empty(shape, device="cuda", dtype=torch.float32)
        st = torch.empty((w.batch, H, D, D), device="cuda", dtype=torch.float32)
        ws_bytes = la.lt_prefill_workspace_bytes(w.batch, w.seqlen, H, D,
                                                 la.LT_F32 if dt == "f32" else la.LT_BF16)
        ws = torch.empty(max(ws_bytes, 1), device="cuda", dtype=torch.uint8)
        call = lambda: la.lt_prefill(q, k, v, slopes, w.block, o=o, state_out=st, workspace=ws,
                                     stream=stream)
        tokens = w.batch * w.seqlen
        nbytes = prefill_bytes(tokens, H, in_bytes=4 if dt == "f32" else 2)
        cfg = {"batch": w.batch, "seq_len": w.seqlen}
    for _ in range(warmup):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"metric": METRIC, "value": round(tokens * steps / wall, 1), "unit": "tokens/s",
            "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": round(wall * 1e3 / steps, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32" if name == "tiny_f32" else "bf16",
            "data": "synthetic",
            "config": dict({"workload": w.name, "heads": H, "head_dim": D, "block": w.block}, **cfg),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                         "bytes_per_launch": nbytes, "kernel": "lt_prefill call"},
            "kernel_ms_mean": round(ms, 5)}


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


def traffic_from(copy_dir, fetch_dir, write_dir, copy_bytes):
    """Per-launch HBM traffic of lt_prefill on the M1 layer from rocprofv3 runs.

    copy_dir holds FETCH_SIZE and WRITE_SIZE of the calibration copy (two runs'
    CSVs may be concatenated there as copy_fetch.csv / copy_write.csv); fetch_dir
    and write_dir hold FETCH_SIZE and WRITE_SIZE of a bench run. Each counter is
    scaled by (bytes the copy moved) / (what the counter read for the copy).
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
    # the plain call's kernels (the counter runs time only plain lt_prefill
    # calls: the norm-gate call and the backward's dq pass plan their pre-pass
    # differently)
    kernels = [k for k in kf if any(n in k for n in ("head_kernel<float, false>", "piece_state_kernel",
                                                      "combine_kernel", "fix_kernel<float, false>"))]
    import numpy as np

    fetch = sum(float(np.median(kf[k])) for k in kernels) * 1024 * f_scale
    write = sum(float(np.median(kw[k])) for k in kernels) * 1024 * w_scale
    out = {"kernel_source_sha256": source_sha(PREFILL_SRCS),
           "kernels": kernels, "fetch_scale": f_scale, "write_scale": w_scale,
           "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write),
           "traffic_bytes_per_launch": round(fetch + write),
           "algorithmic_bytes_per_launch": prefill_bytes(32768, 64)}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def run_cpu_baseline(w, dev_inputs, tokens, min_seconds=10.0, max_reps=50):
    """The fp64 oracle (as it stands) on the host cores, on the first `tokens`
    tokens of the same prefill inputs, all heads; repeated until `min_seconds`
    of CPU work have been timed."""
    import oracle

    q, k, v, slopes = dev_inputs
    hq, hk, hv = (x[:, :tokens].float().cpu().numpy() for x in (q, k, v))
    sl = slopes.cpu().numpy()
    threads = oracle.max_threads()
    reps, dt = 0, 0.0
    while reps < max_reps and (reps == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        oracle.recurrence_batch(hq, hk, hv, sl)
        dt += time.perf_counter() - t0
        reps += 1
    return {"value": round(tokens * reps / dt, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {tokens} of {w.seqlen} tokens, all {w.heads} heads, {reps} runs "
                      f"({reps * tokens * w.heads} (token, head) pairs, {dt:.2f} s, fp64)",
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
    ap.add_argument("--no-norm-gate", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-softmax", action="store_true")
    ap.add_argument("--no-slopes-scaled", action="store_true",
                    help="skip the prefill runs with scaled-down slopes")
    ap.add_argument("--norm-gate-decode-steps", type=int, default=200)
    ap.add_argument("--workload", default="m1_layer",
                    choices=["m1_layer", "long_1m", "varlen", "tiny_f32"])
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--traffic-from", nargs=3, metavar=("COPY_DIR", "FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(*args.traffic_from, args.copy_bytes)
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

    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
        return
    if args.workload != "m1_layer":
        log(f"[bench] {args.workload}")
        print(json.dumps(run_other(la, torch, args.workload, args.steps, args.warmup)), flush=True)
        return

    log("[bench] prefill m1_layer L=32768 H=64 d=128 block=256")
    w, dev_inputs, pre = run_prefill(la, torch, args.steps, args.warmup)
    log(f"[bench] prefill {pre['kernel_ms_mean']:.3f} ms/launch")
    scaled = {}
    for f in (() if args.no_slopes_scaled else (0.1, 1e-5)):
        _, _, r = run_prefill(la, torch, 10, 2, slope_scale=f)
        scaled[f"x{f:g}"] = {"kernel_ms_mean": round(r["kernel_ms_mean"], 5),
                             "tokens_per_s": round(1e3 * w.batch * w.seqlen / r["kernel_ms_mean"], 1),
                             "roofline_frac": r["roofline"]["frac"]}
        log(f"[bench] prefill, slopes x{f:g}: {r['kernel_ms_mean']:.3f} ms/launch")
    dec = None
    if not args.no_decode:
        log(f"[bench] decode batch=256 H=64, {args.decode_steps} steps")
        dec = run_decode(la, torch, args.decode_steps)
        log(f"[bench] decode {dec['ms_per_step_median']:.4f} ms/step")
        dec["slots"] = run_decode(la, torch, args.norm_gate_decode_steps, slots=512)
        log(f"[bench] decode over 512 slots {dec['slots']['ms_per_step_median']:.4f} ms/step")
    ng = None
    if not args.no_norm_gate:
        log("[bench] prefill + norm_gate m1_layer (bf16 gate, bf16 y)")
        ng = {"prefill": run_prefill_norm_gate(la, torch, args.steps, args.warmup)}
        log(f"[bench] prefill + norm_gate {ng['prefill']['kernel_ms_mean']:.3f} ms/launch")
        if not args.no_decode:
            ng["decode"] = run_decode(la, torch, args.norm_gate_decode_steps, norm_gate=True)
            log(f"[bench] decode + norm_gate {ng['decode']['ms_per_step_median']:.4f} ms/step")
    bwd = None
    if not args.no_backward:
        bwd = {}
        for b_, l_ in ((1, 32768), (4, 8192)):
            log(f"[bench] backward batch={b_} L={l_} H=64")
            bwd[f"b{b_}_L{l_}"] = run_backward(la, torch, 10, 2, b_, l_)
            log(f"[bench] backward {bwd[f'b{b_}_L{l_}']['kernel_ms_mean']:.3f} ms/call")
    smx = None
    if not args.no_softmax:
        log("[bench] softmax layer: prefill L=32768 64/8 heads, decode 16 x 32768")
        smx = run_softmax(la, torch, 5, 1, 100)
        log(f"[bench] softmax prefill {smx['prefill']['call_ms_mean']:.3f} ms, decode "
            f"{smx['decode']['ms_per_step_median'] * 1e3:.1f} us")
        if not args.no_cpu:
            log("[bench] softmax oracle on the host")
            sb = run_softmax_cpu_baseline(la, torch)
            smx["prefill"]["cpu_baseline"], smx["decode"]["cpu_baseline"] = sb["prefill"], sb["decode"]
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
        # the same call with every slope scaled down (x0.1: 25 of the 64 heads
        # take the pre-pass; x1e-5: all of them)
        "prefill_slopes_scaled": scaled,
        "decode": dec,
        "norm_gate": ng,
        "backward": bwd,
        "softmax": smx,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
