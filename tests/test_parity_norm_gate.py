"""GPU parity of the norm-gate variants (the operator followed by the
normalisation and gate of the §03 data-flow figure) against the fp64 oracle:
oracle recurrence, then oracle.norm_gate. Relative L2 per (sequence, head) of y
and of the final state: <= 1e-2 for bf16 inputs, <= 1e-5 for fp32 inputs
(decode only; the fused prefill takes bf16)."""

import numpy as np
import pytest

import oracle
import workloads
from parity_util import (TOL_BF16, TOL_F32, ensure_built, max_rel_per_head, max_rel_states,
                         parity_err, to_device, to_host_f32)

pytestmark = pytest.mark.gpu
EPS = workloads.NORM_EPS


@pytest.fixture(scope="module")
def la():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    ensure_built()
    import linear_attention_amd

    return linear_attention_amd


def prefill_ng_case(la, batch, L, H, seed, with_s0=False, out_dtype="f32", workspace="auto"):
    import torch

    print(f"[case] prefill_norm_gate batch={batch} L={L} H={H} seed={seed} s0={with_s0} "
          f"out={out_dtype} ws={workspace}", flush=True)
    q, k, v = workloads.qkv_host(seed, (batch, L, H, 128), "bf16")
    gate = workloads.gate_host(seed + 3, (batch, L, H, 128), "bf16")
    w = workloads.norm_weight_host(seed + 4, H)
    sl = workloads.slopes(H)
    s0 = workloads.state_host(seed + 7, (batch, H, 128, 128)) if with_s0 else None
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    kw = {}
    if workspace == "none":
        kw["workspace"] = torch.empty(0, device="cuda", dtype=torch.uint8)
    y, st = la.lt_prefill_norm_gate(to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"),
                                    torch.from_numpy(sl).cuda(), to_device(gate, "bf16"),
                                    torch.from_numpy(w).cuda(), EPS, 256,
                                    None if s0 is None else torch.from_numpy(s0).cuda(),
                                    out_dtype=od, **kw)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, sl, s0=s0)
    y_ref = oracle.norm_gate(o_ref, gate, w, EPS)
    cu = np.arange(batch + 1) * L
    ey = max_rel_per_head(to_host_f32(y).reshape(batch * L, H, 128), y_ref.reshape(batch * L, H, 128), cu)
    es = max_rel_states(to_host_f32(st), s_ref)
    print(f"[result] y {ey:.3e} state {es:.3e}", flush=True)
    return ey, es


@pytest.mark.parametrize("batch,L,H", [(1, 1, 2), (1, 65, 3), (1, 1000, 4), (2, 333, 3)])
def test_prefill_norm_gate_whole_head(la, batch, L, H):
    """Short inputs with fewer than 256 (sequence, head) pairs: one workgroup
    per pair (the plain prefill would split value columns here)."""
    ey, es = prefill_ng_case(la, batch, L, H, 700 + L)
    assert ey <= TOL_BF16 and es <= TOL_BF16


@pytest.mark.parametrize("L,H,with_s0", [(9000, 1, False), (5000, 2, True), (20000, 3, False)])
def test_prefill_norm_gate_segmented(la, L, H, with_s0):
    ey, es = prefill_ng_case(la, 1, L, H, 800 + L, with_s0=with_s0)
    assert ey <= TOL_BF16 and es <= TOL_BF16


def test_prefill_norm_gate_bf16_output_and_no_workspace(la):
    ey, es = prefill_ng_case(la, 1, 6000, 2, 901, out_dtype="bf16", workspace="none")
    assert ey <= TOL_BF16 and es <= TOL_BF16


def test_prefill_norm_gate_many_pairs(la):
    """256 or more (sequence, head) pairs: whole heads, no segments."""
    ey, es = prefill_ng_case(la, 4, 700, 64, 902, with_s0=True)
    assert ey <= TOL_BF16 and es <= TOL_BF16


def test_prefill_norm_gate_in_place_state(la):
    import torch

    L, H = 9000, 2
    q, k, v = workloads.qkv_host(903, (1, L, H, 128), "bf16")
    gate = workloads.gate_host(904, (1, L, H, 128), "bf16")
    w = workloads.norm_weight_host(905, H)
    sl = workloads.slopes(H)
    s0 = workloads.state_host(906, (1, H, 128, 128))
    st = torch.from_numpy(s0).cuda()
    y, _ = la.lt_prefill_norm_gate(to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"),
                                   torch.from_numpy(sl).cuda(), to_device(gate, "bf16"),
                                   torch.from_numpy(w).cuda(), EPS, 256, st, state_out=st)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, sl, s0=s0)
    y_ref = oracle.norm_gate(o_ref, gate, w, EPS)
    ey = max(parity_err(to_host_f32(y)[0, :, h], y_ref[0, :, h]) for h in range(H))
    es = max_rel_states(to_host_f32(st), s_ref)
    assert ey <= TOL_BF16 and es <= TOL_BF16, (ey, es)


def test_prefill_varlen_norm_gate(la):
    import torch

    lens = np.array([300, 0, 1, 2100, 64, 4500], np.int64)
    cu = workloads.cu_seqlens(lens)
    T, H = int(cu[-1]), 3
    print(f"[case] varlen_norm_gate T={T} lens={list(lens)}", flush=True)
    q, k, v = workloads.qkv_host(910, (T, H, 128), "bf16")
    gate = workloads.gate_host(911, (T, H, 128), "bf16")
    w = workloads.norm_weight_host(912, H)
    sl = workloads.slopes(H)
    s0 = workloads.state_host(913, (len(lens), H, 128, 128))
    y, st = la.lt_prefill_varlen_norm_gate(
        to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"), torch.from_numpy(cu).cuda(),
        torch.from_numpy(sl).cuda(), to_device(gate, "bf16"), torch.from_numpy(w).cuda(), EPS, 256,
        torch.from_numpy(s0).cuda())
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence_packed(q, k, v, sl, cu, s0=s0)
    y_ref = oracle.norm_gate(o_ref, gate, w, EPS)
    ey = max_rel_per_head(to_host_f32(y), y_ref, cu)
    es = max_rel_states(to_host_f32(st), s_ref)
    print(f"[result] y {ey:.3e} state {es:.3e}", flush=True)
    assert ey <= TOL_BF16 and es <= TOL_BF16


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_norm_gate_steps(la, dtype):
    """Five decode steps from a carried state; every step's y and the final state."""
    import torch

    B, H, steps = 6, 5, 5
    print(f"[case] decode_norm_gate B={B} H={H} dtype={dtype}", flush=True)
    s0 = workloads.state_host(920, (B, H, 128, 128))
    w = workloads.norm_weight_host(921, H)
    sl = workloads.slopes(H)
    state = torch.from_numpy(s0).cuda()
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    st_ref = s0.astype(np.float64)
    worst = 0.0
    for t in range(steps):
        q, k, v = workloads.qkv_host(930 + t, (B, H, 128), dtype)
        gate = workloads.gate_host(940 + t, (B, H, 128), dtype)
        y = la.lt_decode_norm_gate(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype),
                                   torch.from_numpy(sl).cuda(), state, to_device(gate, dtype),
                                   torch.from_numpy(w).cuda(), EPS)
        torch.cuda.synchronize()
        o_ref, st_ref = oracle.decode(q, k, v, sl, st_ref)
        y_ref = oracle.norm_gate(o_ref, gate, w, EPS)
        yg = to_host_f32(y)
        worst = max(worst, max(parity_err(yg[b, h], y_ref[b, h]) for b in range(B) for h in range(H)))
    es = max_rel_states(to_host_f32(state), st_ref)
    print(f"[result] y {worst:.3e} state {es:.3e}", flush=True)
    assert worst <= tol and es <= tol


def test_decode_norm_gate_bf16_output(la):
    import torch

    B, H = 3, 4
    q, k, v = workloads.qkv_host(950, (B, H, 128), "bf16")
    gate = workloads.gate_host(951, (B, H, 128), "bf16")
    w = workloads.norm_weight_host(952, H)
    sl = workloads.slopes(H)
    s0 = workloads.state_host(953, (B, H, 128, 128))
    state = torch.from_numpy(s0).cuda()
    y = la.lt_decode_norm_gate(to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"),
                               torch.from_numpy(sl).cuda(), state, to_device(gate, "bf16"),
                               torch.from_numpy(w).cuda(), EPS, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    o_ref, _ = oracle.decode(q, k, v, sl, s0)
    y_ref = oracle.norm_gate(o_ref, gate, w, EPS)
    yg = to_host_f32(y)
    assert max(parity_err(yg[b, h], y_ref[b, h]) for b in range(B) for h in range(H)) <= TOL_BF16


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_prefill_norm_gate_segmented_slope_mix(la, out_dtype):
    """Norm-gate prefill of the segmented plan over heads on both routes: the
    short-memory heads (0.02, 0.2, 1, 30) take warm-up ranges (each range
    rebuilds its carried-in state from the tokens just before it), 0 and 1e-6
    the pre-pass. Carried-in state updated in place, so the warm-up heads'
    final states go through the workspace."""
    import torch

    L, H = 9000, 6
    sl = np.array([0.0, 1e-6, 0.02, 0.2, 1.0, 30.0], np.float32)
    print(f"[case] norm-gate segmented slope mix L={L} slopes={list(sl)} out={out_dtype}", flush=True)
    q, k, v = workloads.qkv_host(2401, (1, L, H, 128), "bf16")
    gate = workloads.gate_host(2402, (1, L, H, 128), "bf16")
    w = workloads.norm_weight_host(2403, H)
    s0 = workloads.state_host(2404, (1, H, 128, 128))
    st = torch.from_numpy(s0).cuda()
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    y, _ = la.lt_prefill_norm_gate(to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"),
                                   torch.from_numpy(sl).cuda(), to_device(gate, "bf16"),
                                   torch.from_numpy(w).cuda(), EPS, 256, st, state_out=st, out_dtype=od)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, sl, s0=s0)
    y_ref = oracle.norm_gate(o_ref, gate, w, EPS)
    yg = to_host_f32(y)
    ey = max(parity_err(yg[0, :, h], y_ref[0, :, h]) for h in range(H))
    es = max_rel_states(to_host_f32(st), s_ref)
    print(f"[result] y {ey:.3e} state {es:.3e}", flush=True)
    assert ey <= TOL_BF16 and es <= TOL_BF16, (ey, es)


def test_prefill_norm_gate_segmented_no_final_state(la):
    """Segmented norm-gate prefill over warm-up heads only, with no final state
    requested."""
    import torch

    L, H = 9000, 4
    sl = np.array([0.02, 0.2, 1.0, 30.0], np.float32)
    print(f"[case] norm-gate segmented, no state_out, L={L} slopes={list(sl)}", flush=True)
    q, k, v = workloads.qkv_host(2411, (1, L, H, 128), "bf16")
    gate = workloads.gate_host(2412, (1, L, H, 128), "bf16")
    w = workloads.norm_weight_host(2413, H)
    s0 = workloads.state_host(2414, (1, H, 128, 128))
    y, st = la.lt_prefill_norm_gate(to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"),
                                    torch.from_numpy(sl).cuda(), to_device(gate, "bf16"),
                                    torch.from_numpy(w).cuda(), EPS, 256, torch.from_numpy(s0).cuda(),
                                    want_state=False, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert st is None
    o_ref, _ = oracle.recurrence_batch(q, k, v, sl, s0=s0)
    y_ref = oracle.norm_gate(o_ref, gate, w, EPS)
    yg = to_host_f32(y)
    ey = max(parity_err(yg[0, :, h], y_ref[0, :, h]) for h in range(H))
    print(f"[result] y {ey:.3e}", flush=True)
    assert ey <= TOL_BF16, ey


def test_prefill_norm_gate_segmented_batch(la):
    """Segmented norm-gate prefill with several sequences (3 x 9000 tokens, 4
    heads on both routes), carried-in states, fp32 y."""
    import torch

    B, L, H = 3, 9000, 4
    sl = np.array([1e-6, 0.02, 0.3, 4.0], np.float32)
    print(f"[case] norm-gate segmented batch={B} L={L} slopes={list(sl)}", flush=True)
    q, k, v = workloads.qkv_host(2421, (B, L, H, 128), "bf16")
    gate = workloads.gate_host(2422, (B, L, H, 128), "bf16")
    w = workloads.norm_weight_host(2423, H)
    s0 = workloads.state_host(2424, (B, H, 128, 128))
    y, st = la.lt_prefill_norm_gate(to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"),
                                    torch.from_numpy(sl).cuda(), to_device(gate, "bf16"),
                                    torch.from_numpy(w).cuda(), EPS, 256, torch.from_numpy(s0).cuda())
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, sl, s0=s0)
    y_ref = oracle.norm_gate(o_ref, gate, w, EPS)
    yg = to_host_f32(y)
    ey = max(parity_err(yg[b, :, h], y_ref[b, :, h]) for b in range(B) for h in range(H))
    es = max_rel_states(to_host_f32(st), s_ref)
    print(f"[result] y {ey:.3e} state {es:.3e}", flush=True)
    assert ey <= TOL_BF16 and es <= TOL_BF16, (ey, es)
