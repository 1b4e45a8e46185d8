"""GPU parity at the full sizes of the benchmark workloads, in the launch
configuration the benchmark times.

  * M1 Lightning layer: batch 1, 32768 tokens, 64 heads x 128, block 256, bf16;
    every head's output and final state against the oracle.
  * 1M-token prefill: batch 1, 2^20 tokens, 64 heads; output and final state on
    sampled heads {0, 21, 42, 63} (fastest to slowest decay).
  * Batched decode: 256 sequences x 64 heads, 1000 steps; the carried-in states
    of sampled sequences are oracle prefill states of 4096 random bf16 tokens;
    every step's output of the sampled sequences and their final states; and a
    short run checking every (sequence, head) state.
  * Varlen prefill: 16 sequences of 1024..65536 tokens with N(0, 0.01) carried-in
    states; every final state, and outputs on sampled heads.

Relative L2 per (sequence, head) <= 1e-2 (bf16 inputs), and every output row
within 5e-2 of the head's RMS row norm (parity_util.parity_err); the rows next
to the segmented plan's switches are also reported on their own.
"""

import numpy as np
import pytest

import oracle
import workloads
from parity_util import TOL_BF16, ensure_built, parity_err, segment_boundary_err, to_host_f32

pytestmark = pytest.mark.gpu

SAMPLED_HEADS = [0, 21, 42, 63]


@pytest.fixture(scope="module")
def la():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    ensure_built()
    import linear_attention_amd

    return linear_attention_amd


def head_slice(x, h):
    """[1, L, H, d] or [T, H, d] device tensor -> host float32 [L, d] of head h."""
    return to_host_f32(x[..., h, :].contiguous()).reshape(-1, x.shape[-1])


def test_m1_layer_all_heads(la):
    import torch

    w = workloads.M1_LAYER
    print(f"[case] {w.name} L={w.seqlen} H={w.heads}", flush=True)
    q, k, v = workloads.qkv_device(w.seed, (1, w.seqlen, w.heads, 128), "bf16")
    sl = workloads.slopes(w.heads)
    o, st = la.lt_prefill(q, k, v, torch.from_numpy(sl).cuda(), w.block)
    torch.cuda.synchronize()
    hq, hk, hv = (to_host_f32(x) for x in (q, k, v))
    o_ref, s_ref = oracle.recurrence_batch(hq, hk, hv, sl)
    o_g, s_g = to_host_f32(o), to_host_f32(st)
    worst_o = max(parity_err(o_g[0, :, h], o_ref[0, :, h]) for h in range(w.heads))
    worst_s = max(parity_err(s_g[0, h], s_ref[0, h]) for h in range(w.heads))
    worst_b = max(segment_boundary_err(o_g[0, :, h], o_ref[0, :, h], 1, w.seqlen, w.heads, sl[h])
                  for h in range(w.heads))
    print(f"[result] worst parity err: o {worst_o:.3e} state {worst_s:.3e} "
          f"segment-boundary rows {worst_b:.3e}", flush=True)
    assert worst_o <= TOL_BF16 and worst_s <= TOL_BF16 and worst_b <= TOL_BF16


def test_m1_layer_norm_gate_all_heads(la):
    """The M1 layer through lt_prefill_norm_gate (bf16 gate and y), every head."""
    import torch

    w = workloads.M1_LAYER
    print(f"[case] {w.name} norm_gate L={w.seqlen} H={w.heads}", flush=True)
    shape = (1, w.seqlen, w.heads, 128)
    q, k, v = workloads.qkv_device(w.seed, shape, "bf16")
    gate = workloads.gate_device(w.seed + 10, shape, "bf16")
    nw = workloads.norm_weight_host(w.seed + 11, w.heads)
    sl = workloads.slopes(w.heads)
    y, st = la.lt_prefill_norm_gate(q, k, v, torch.from_numpy(sl).cuda(), gate,
                                    torch.from_numpy(nw).cuda(), workloads.NORM_EPS, w.block,
                                    out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    hq, hk, hv = (to_host_f32(x) for x in (q, k, v))
    o_ref, s_ref = oracle.recurrence_batch(hq, hk, hv, sl)
    y_ref = oracle.norm_gate(o_ref, to_host_f32(gate), nw, workloads.NORM_EPS)
    y_g, s_g = to_host_f32(y), to_host_f32(st)
    worst_y = max(parity_err(y_g[0, :, h], y_ref[0, :, h]) for h in range(w.heads))
    worst_s = max(parity_err(s_g[0, h], s_ref[0, h]) for h in range(w.heads))
    print(f"[result] worst rel L2: y {worst_y:.3e} state {worst_s:.3e}", flush=True)
    assert worst_y <= TOL_BF16 and worst_s <= TOL_BF16


def test_m1_layer_backward_all_heads(la):
    """lt_prefill_backward on the M1 layer (batch 1, 32768 tokens, 64 heads, fp32
    gradients, with a final-state gradient), every head against the oracle."""
    import torch

    w = workloads.M1_LAYER
    print(f"[case] {w.name} backward L={w.seqlen} H={w.heads}", flush=True)
    shape = (1, w.seqlen, w.heads, 128)
    q, k, v = workloads.qkv_device(w.seed, shape, "bf16")
    do = workloads.gate_device(w.seed + 20, shape, "bf16")
    ds = workloads.state_device(w.seed + 21, (1, w.heads, 128, 128), std=0.1)
    sl = workloads.slopes(w.heads)
    dq, dk, dv, dsi = la.lt_prefill_backward(q, k, v, do, torch.from_numpy(sl).cuda(), w.block,
                                             None, ds)
    torch.cuda.synchronize()
    hq, hk, hv, hdo = (to_host_f32(x) for x in (q, k, v, do))
    rq, rk, rv, rs = oracle.backward_batch(hq, hk, hv, hdo, sl, ds=to_host_f32(ds))
    worst = {}
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        gh = to_host_f32(g)
        worst[name] = max(parity_err(gh[0, :, h], r[0, :, h]) for h in range(w.heads))
    sg = to_host_f32(dsi)
    worst["ds0"] = max(parity_err(sg[0, h], rs[0, h]) for h in range(w.heads))
    print(f"[result] worst rel L2 {worst}", flush=True)
    assert max(worst.values()) <= TOL_BF16


def test_long_context_1m_sampled_heads(la):
    import torch

    w = workloads.LONG_1M
    print(f"[case] {w.name} L={w.seqlen} H={w.heads} heads={SAMPLED_HEADS}", flush=True)
    q, k, v = workloads.qkv_device(w.seed, (1, w.seqlen, w.heads, 128), "bf16")
    sl = workloads.slopes(w.heads)
    o, st = la.lt_prefill(q, k, v, torch.from_numpy(sl).cuda(), w.block)
    torch.cuda.synchronize()
    hs = SAMPLED_HEADS
    hq = np.stack([head_slice(q, h) for h in hs], axis=1)[None]  # [1, L, 4, d]
    hk = np.stack([head_slice(k, h) for h in hs], axis=1)[None]
    hv = np.stack([head_slice(v, h) for h in hs], axis=1)[None]
    del q, k, v
    o_ref, s_ref = oracle.recurrence_batch(hq, hk, hv, sl[hs])
    s_g = to_host_f32(st)
    for j, h in enumerate(hs):
        og = head_slice(o, h)
        eo = parity_err(og, o_ref[0, :, j])
        es = parity_err(s_g[0, h], s_ref[0, j])
        eb = segment_boundary_err(og, o_ref[0, :, j], 1, w.seqlen, w.heads, sl[h])
        print(f"[result] head {h}: o {eo:.3e} state {es:.3e} segment-boundary rows {eb:.3e}",
              flush=True)
        assert eo <= TOL_BF16 and es <= TOL_BF16 and eb <= TOL_BF16


def _history_states(seed, seqs, H, d, history):
    """Oracle prefill states after `history` random bf16 tokens for the sampled
    sequences (one independent stream per sequence)."""
    sl = workloads.slopes(H)
    out = np.zeros((len(seqs), H, d, d), np.float64)
    children = np.random.SeedSequence(seed).spawn(max(seqs) + 1)
    for j, s in enumerate(seqs):
        g = np.random.Generator(np.random.PCG64(children[s]))
        x = [workloads.round_bf16(g.standard_normal((1, history, H, d), dtype=np.float32)
                                  * np.float32(workloads.INPUT_SCALE)) for _ in range(3)]
        _, st = oracle.recurrence_batch(x[0], x[1], x[2], sl, want_o=False)
        out[j] = st[0]
    return out


def test_batched_decode_1000_steps_sampled_sequences(la):
    import torch

    w = workloads.DECODE
    B, H, d, steps = w.batch, w.heads, 128, w.extra["steps"]
    seqs = [0, 37, 85, 128, 170, 201, 233, 255]
    print(f"[case] {w.name} B={B} H={H} steps={steps} sampled={seqs}", flush=True)
    s0_sampled = _history_states(w.seed, seqs, H, d, w.extra["history"])
    state = workloads.state_device(w.seed + 2, (B, H, d, d), std=0.05)
    state[seqs] = torch.from_numpy(s0_sampled.astype(np.float32)).cuda()
    s0_host = to_host_f32(state[seqs])  # the fp32 states the GPU starts from
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed + 1)
    qkv = (torch.randn((steps, 3, B, H, d), generator=g, device="cuda")
           .mul_(workloads.INPUT_SCALE).to(torch.bfloat16))
    slopes = torch.from_numpy(workloads.slopes(H)).cuda()
    idx = torch.tensor(seqs, device="cuda")
    o_hist = torch.empty((steps, len(seqs), H, d), device="cuda", dtype=torch.float32)
    o = torch.empty((B, H, d), device="cuda", dtype=torch.float32)
    for t in range(steps):
        la.lt_decode(qkv[t, 0], qkv[t, 1], qkv[t, 2], slopes, state, o=o)
        o_hist[t] = o.index_select(0, idx)
    torch.cuda.synchronize()
    hq = to_host_f32(qkv[:, 0].index_select(1, idx)).transpose(1, 0, 2, 3)  # [seqs, steps, H, d]
    hk = to_host_f32(qkv[:, 1].index_select(1, idx)).transpose(1, 0, 2, 3)
    hv = to_host_f32(qkv[:, 2].index_select(1, idx)).transpose(1, 0, 2, 3)
    o_ref, s_ref = oracle.recurrence_batch(hq, hk, hv, workloads.slopes(H), s0=s0_host)
    og = to_host_f32(o_hist)  # [steps, seqs, H, d]
    worst_o = 0.0
    for j in range(len(seqs)):
        for h in range(H):
            worst_o = max(worst_o, parity_err(og[:, j, h], o_ref[j, :, h]))
    sg = to_host_f32(state[seqs])
    worst_s = max(parity_err(sg[j, h], s_ref[j, h]) for j in range(len(seqs)) for h in range(H))
    # per-step check on the worst (sequence, head) as well
    step_worst = max(parity_err(og[t, j, h], o_ref[j, t, h]) for t in (0, steps // 2, steps - 1)
                     for j in range(len(seqs)) for h in range(H))
    print(f"[result] o {worst_o:.3e} (single steps {step_worst:.3e}) state {worst_s:.3e}",
          flush=True)
    assert worst_o <= TOL_BF16 and worst_s <= TOL_BF16 and step_worst <= TOL_BF16


def test_batched_decode_all_units_short(la):
    """Every (sequence, head) of the 256 x 64 decode batch over 8 steps."""
    import torch

    B, H, d, steps = 256, 64, 128, 8
    print(f"[case] decode all units B={B} H={H} steps={steps}", flush=True)
    state = workloads.state_device(4104, (B, H, d, d), std=0.05)
    s0 = to_host_f32(state)
    g = torch.Generator(device="cuda")
    g.manual_seed(4105)
    qkv = (torch.randn((steps, 3, B, H, d), generator=g, device="cuda")
           .mul_(workloads.INPUT_SCALE).to(torch.bfloat16))
    slopes = torch.from_numpy(workloads.slopes(H)).cuda()
    outs = []
    for t in range(steps):
        outs.append(la.lt_decode(qkv[t, 0], qkv[t, 1], qkv[t, 2], slopes, state))
    torch.cuda.synchronize()
    h = to_host_f32(qkv).transpose(1, 2, 0, 3, 4)  # [3, B, steps, H, d]
    o_ref, s_ref = oracle.recurrence_batch(h[0], h[1], h[2], workloads.slopes(H), s0=s0)
    sg = to_host_f32(state)
    worst_s = max(parity_err(sg[b, hh], s_ref[b, hh]) for b in range(B) for hh in range(H))
    og = np.stack([to_host_f32(x) for x in outs], axis=1)  # [B, steps, H, d]
    worst_o = max(parity_err(og[b, :, hh], o_ref[b, :, hh]) for b in range(B) for hh in range(H))
    print(f"[result] o {worst_o:.3e} state {worst_s:.3e}", flush=True)
    assert worst_o <= TOL_BF16 and worst_s <= TOL_BF16


def test_varlen_carried_state(la):
    import torch

    w = workloads.VARLEN
    lens = workloads.varlen_lengths(w.seed, w.batch, w.extra["min_len"], w.extra["max_len"])
    cu = workloads.cu_seqlens(lens)
    T, H, d = int(cu[-1]), w.heads, 128
    print(f"[case] {w.name} T={T} lens={list(lens)}", flush=True)
    q, k, v = workloads.qkv_device(w.seed, (T, H, d), "bf16")
    s0 = workloads.state_device(w.seed + 1, (len(lens), H, d, d), std=0.1)
    sl = workloads.slopes(H)
    o, st = la.lt_prefill_varlen(q, k, v, torch.from_numpy(cu).cuda(), torch.from_numpy(sl).cuda(),
                                 w.block, s0)
    torch.cuda.synchronize()
    s0h = to_host_f32(s0)
    sg = to_host_f32(st)
    # final states of every (sequence, head): state-only oracle, 8 heads at a time
    worst_s = 0.0
    for h0 in range(0, H, 8):
        hs = list(range(h0, h0 + 8))
        kh = to_host_f32(k[:, h0:h0 + 8].contiguous())
        vh = to_host_f32(v[:, h0:h0 + 8].contiguous())
        _, s_ref = oracle.recurrence_packed(kh, kh, vh, sl[hs], cu, s0=s0h[:, hs], want_o=False)
        worst_s = max(worst_s, max(parity_err(sg[n, h0 + j], s_ref[n, j])
                                   for n in range(len(lens)) for j in range(8)))
    # outputs on sampled heads
    hs = SAMPLED_HEADS
    qh = to_host_f32(q[:, hs].contiguous())
    kh = to_host_f32(k[:, hs].contiguous())
    vh = to_host_f32(v[:, hs].contiguous())
    o_ref, _ = oracle.recurrence_packed(qh, kh, vh, sl[hs], cu, s0=s0h[:, hs])
    og = to_host_f32(o[:, hs].contiguous())
    worst_o = 0.0
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        for j in range(len(hs)):
            worst_o = max(worst_o, parity_err(og[a:b, j], o_ref[a:b, j]))
    print(f"[result] o {worst_o:.3e} state {worst_s:.3e}", flush=True)
    assert worst_o <= TOL_BF16 and worst_s <= TOL_BF16
