"""GPU parity of lt_prefill_backward against the fp64 oracle backward
(oracle.backward_batch): dq, dk, dv per (sequence, head) and d_state_in, relative
L2 <= 1e-2 (bf16 inputs)."""

import numpy as np
import pytest

import oracle
import workloads
from parity_util import TOL_BF16, ensure_built, max_rel_states, parity_err, to_device, to_host_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def la():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    ensure_built()
    import linear_attention_amd

    return linear_attention_amd


def backward_case(la, batch, L, H, seed, with_state=False, grad_dtype="f32", workspace="auto"):
    import torch

    print(f"[case] backward batch={batch} L={L} H={H} seed={seed} state={with_state} "
          f"grad={grad_dtype} ws={workspace}", flush=True)
    q, k, v = workloads.qkv_host(seed, (batch, L, H, 128), "bf16")
    do = workloads.gate_host(seed + 1, (batch, L, H, 128), "bf16")  # N(0, 1) bf16
    sl = workloads.slopes(H)
    s0 = workloads.state_host(seed + 2, (batch, H, 128, 128)) if with_state else None
    ds = workloads.state_host(seed + 3, (batch, H, 128, 128)) if with_state else None
    gd = torch.float32 if grad_dtype == "f32" else torch.bfloat16
    dq, dk, dv, dsi = la.lt_prefill_backward(
        to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"), to_device(do, "bf16"),
        torch.from_numpy(sl).cuda(), 256, None if s0 is None else torch.from_numpy(s0).cuda(),
        None if ds is None else torch.from_numpy(ds).cuda(), grad_dtype=gd,
        **({"workspace": torch.empty(0, device="cuda", dtype=torch.uint8)} if workspace == "none" else {}))
    torch.cuda.synchronize()
    rq, rk, rv, rs = oracle.backward_batch(q, k, v, do, sl, s0=s0, ds=ds)
    errs = {}
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        gh = to_host_f32(g)
        errs[name] = max(parity_err(gh[b, :, h], r[b, :, h]) for b in range(batch) for h in range(H))
    errs["ds0"] = max_rel_states(to_host_f32(dsi), rs)
    print(f"[result] {errs}", flush=True)
    return errs


@pytest.mark.parametrize("L", [1, 63, 64, 65, 200])
def test_backward_lengths(la, L):
    errs = backward_case(la, 1, L, 2, 1300 + L)
    assert max(errs.values()) <= TOL_BF16, errs


def test_backward_batch_and_state(la):
    errs = backward_case(la, 3, 190, 3, 1401, with_state=True)
    assert max(errs.values()) <= TOL_BF16, errs


@pytest.mark.parametrize("L,H", [(9000, 1), (5000, 2), (20000, 3), (16384, 4)])
def test_backward_long_sequences(la, L, H):
    """Long sequences with few heads: the dq pass takes the segmented forward
    plan and the reverse pass its mirrored segments (pieces with boundaries
    inside and at their ends)."""
    errs = backward_case(la, 1, L, H, 1500 + L, with_state=True)
    assert max(errs.values()) <= TOL_BF16, errs


def test_backward_many_pairs(la):
    errs = backward_case(la, 4, 700, 64, 1601)
    assert max(errs.values()) <= TOL_BF16, errs


def test_backward_bf16_gradients(la):
    errs = backward_case(la, 2, 300, 2, 1701, with_state=True, grad_dtype="bf16")
    assert max(errs.values()) <= TOL_BF16, errs


def test_backward_zero_length_passes_state_gradient(la):
    import torch

    H = 2
    ds = workloads.state_host(1801, (1, H, 128, 128))
    z = torch.empty((1, 0, H, 128), device="cuda", dtype=torch.bfloat16)
    _, _, _, dsi = la.lt_prefill_backward(z, z, z, z, torch.from_numpy(workloads.slopes(H)).cuda(),
                                          64, None, torch.from_numpy(ds).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(to_host_f32(dsi), ds)


def test_backward_long_sequence_without_workspace(la):
    """No workspace: one workgroup per (sequence, head) in both passes."""
    errs = backward_case(la, 1, 9000, 2, 1901, with_state=True, workspace="none")
    assert max(errs.values()) <= TOL_BF16, errs


@pytest.mark.parametrize("grad_dtype", ["f32", "bf16"])
def test_backward_segmented_slope_mix(la, grad_dtype):
    """Segmented backward over heads on both routes of both passes: short-memory
    heads (slopes 0.012, 0.02, 0.2, 1, 30) on warm-up ranges (warm-ups of 1,024,
    640 and 128 tokens, against 2,304-token segments; the reverse pass's ranges
    and fine chunks are cut from the end of the sequence, so its last piece
    holds the ragged first 9000 mod 64 tokens), 0 and 1e-6 on the pre-passes;
    carried-in state and final-state gradient."""
    import torch

    L, H = 9000, 7
    sl = np.array([0.0, 1e-6, 0.012, 0.02, 0.2, 1.0, 30.0], np.float32)
    print(f"[case] backward segmented slope mix L={L} slopes={list(sl)} grad={grad_dtype}", flush=True)
    q, k, v = workloads.qkv_host(2501, (1, L, H, 128), "bf16")
    do = workloads.gate_host(2502, (1, L, H, 128), "bf16")
    s0 = workloads.state_host(2503, (1, H, 128, 128))
    ds = workloads.state_host(2504, (1, H, 128, 128))
    gd = torch.float32 if grad_dtype == "f32" else torch.bfloat16
    dq, dk, dv, dsi = la.lt_prefill_backward(
        to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"), to_device(do, "bf16"),
        torch.from_numpy(sl).cuda(), 256, torch.from_numpy(s0).cuda(), torch.from_numpy(ds).cuda(), grad_dtype=gd)
    torch.cuda.synchronize()
    rq, rk, rv, rs = oracle.backward_batch(q, k, v, do, sl, s0=s0, ds=ds)
    errs = {}
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        gh = to_host_f32(g)
        errs[name] = max(parity_err(gh[0, :, h], r[0, :, h]) for h in range(H))
    errs["ds0"] = max_rel_states(to_host_f32(dsi), rs)
    print(f"[result] {errs}", flush=True)
    assert max(errs.values()) <= TOL_BF16, errs


def test_backward_prepass_groups(la):
    """Backward with every head on both pre-passes (48 heads, slopes scaled by
    1e-4; 10240 tokens: 16 pieces merged into groups of 3, counted from the
    end, the last of one piece, one group ending on a segment boundary):
    sampled heads against the oracle, with carried state and final-state
    gradient."""
    import torch

    L, H = 10240, 48
    sl = (workloads.slopes(H) * np.float32(1e-4)).astype(np.float32)
    print(f"[case] backward pre-pass groups L={L} H={H}", flush=True)
    q, k, v = workloads.qkv_host(2521, (1, L, H, 128), "bf16")
    do = workloads.gate_host(2522, (1, L, H, 128), "bf16")
    s0 = workloads.state_host(2523, (1, H, 128, 128))
    ds = workloads.state_host(2524, (1, H, 128, 128))
    dq, dk, dv, dsi = la.lt_prefill_backward(
        to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"), to_device(do, "bf16"),
        torch.from_numpy(sl).cuda(), 256, torch.from_numpy(s0).cuda(), torch.from_numpy(ds).cuda())
    torch.cuda.synchronize()
    hs = [0, 5, 33, 47]
    sub = lambda x: np.ascontiguousarray(x[:, :, hs])
    rq, rk, rv, rs = oracle.backward_batch(sub(q), sub(k), sub(v), sub(do), np.ascontiguousarray(sl[hs]),
                                           s0=np.ascontiguousarray(s0[:, hs]), ds=np.ascontiguousarray(ds[:, hs]))
    errs = {}
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        gh = to_host_f32(g)[:, :, hs]
        errs[name] = max(parity_err(gh[0, :, i], r[0, :, i]) for i in range(len(hs)))
    errs["ds0"] = max_rel_states(to_host_f32(dsi)[:, hs], rs)
    print(f"[result] {errs}", flush=True)
    assert max(errs.values()) <= TOL_BF16, errs


def test_backward_segmented_batch_slope_mix(la):
    """Segmented backward with several sequences (2 x 9000 tokens, 4 heads) over
    heads on both routes of both passes, with carried state and final-state
    gradient."""
    import torch

    B, L, H = 2, 9000, 4
    sl = np.array([0.0, 0.01, 0.3, 4.0], np.float32)
    print(f"[case] backward segmented batch={B} L={L} slopes={list(sl)}", flush=True)
    q, k, v = workloads.qkv_host(2531, (B, L, H, 128), "bf16")
    do = workloads.gate_host(2532, (B, L, H, 128), "bf16")
    s0 = workloads.state_host(2533, (B, H, 128, 128))
    ds = workloads.state_host(2534, (B, H, 128, 128))
    assert la.lt_prefill_workspace_bytes(B, L, H) > 0
    dq, dk, dv, dsi = la.lt_prefill_backward(
        to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"), to_device(do, "bf16"),
        torch.from_numpy(sl).cuda(), 256, torch.from_numpy(s0).cuda(), torch.from_numpy(ds).cuda())
    torch.cuda.synchronize()
    rq, rk, rv, rs = oracle.backward_batch(q, k, v, do, sl, s0=s0, ds=ds)
    errs = {}
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        gh = to_host_f32(g)
        errs[name] = max(parity_err(gh[b, :, h], r[b, :, h]) for b in range(B) for h in range(H))
    errs["ds0"] = max_rel_states(to_host_f32(dsi), rs)
    print(f"[result] {errs}", flush=True)
    assert max(errs.values()) <= TOL_BF16, errs
