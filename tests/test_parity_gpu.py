"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small and medium shapes that span several 64-token sub-blocks, ragged tails,
empty inputs, carried-in states, in-place state updates, both input dtypes and
both output dtypes. Tolerance: relative L2 per (sequence, head) of O and of
the final state, <= 1e-5 for fp32 inputs and <= 1e-2 for bf16 inputs, and
every row (token, or key row of a state) within 5x that of the slice's RMS row
norm (parity_util.parity_err).
"""

import numpy as np
import pytest

import oracle
import workloads
from parity_util import (TOL_BF16, TOL_F32, ensure_built, max_rel_per_head, max_rel_states,
                         parity_err, segment_boundary_err, to_device, to_host_f32)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def la():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    ensure_built()
    import linear_attention_amd

    return linear_attention_amd


def tol(dtype):
    return TOL_F32 if dtype == "f32" else TOL_BF16


def run_prefill_case(la, batch, L, H, dtype, seed, block=256, with_s0=False, out_dtype="f32"):
    import torch

    print(f"[case] prefill batch={batch} L={L} H={H} dtype={dtype} seed={seed} s0={with_s0}",
          flush=True)
    q, k, v = workloads.qkv_host(seed, (batch, L, H, 128), dtype)
    sl = workloads.slopes(H)
    s0 = workloads.state_host(seed + 7, (batch, H, 128, 128)) if with_s0 else None
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    o, st = la.lt_prefill(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype),
                          torch.from_numpy(sl).cuda(), block,
                          None if s0 is None else torch.from_numpy(s0).cuda(), out_dtype=od)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, sl, s0=s0)
    o_g, s_g = to_host_f32(o), to_host_f32(st)
    cu = np.arange(batch + 1) * L
    eo = max_rel_per_head(o_g.reshape(batch * L, H, 128), o_ref.reshape(batch * L, H, 128), cu)
    es = max_rel_states(s_g, s_ref)
    if L > 0 and dtype == "bf16":  # the rows next to the plan's switches, on their own
        eb = max(segment_boundary_err(o_g[b, :, h], o_ref[b, :, h], batch, L, H, sl[h])
                 for b in range(batch) for h in range(H))
        print(f"[result] o {eo:.3e} state {es:.3e} segment-boundary rows {eb:.3e}", flush=True)
        eo = max(eo, eb)
    return eo, es


def test_init_loads_and_repeats(la):
    """lt_init succeeds on the device, again on a second call, and a prefill
    after it matches the oracle."""
    print("[case] lt_init twice, then a 300-token prefill", flush=True)
    assert la.lib.lt_init() == la.LT_OK
    la.lt_init()
    eo, es = run_prefill_case(la, 1, 300, 3, "bf16", 1203)
    assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)


@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 128, 200, 1000])
def test_prefill_bf16_lengths(la, L):
    eo, es = run_prefill_case(la, 1, L, 4, "bf16", 100 + L)
    assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)


@pytest.mark.parametrize("L", [1, 63, 64, 65, 300])
def test_prefill_f32_lengths(la, L):
    eo, es = run_prefill_case(la, 1, L, 4, "f32", 200 + L)
    assert eo <= TOL_F32 and es <= TOL_F32, (eo, es)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_batch_and_carried_state(la, dtype):
    eo, es = run_prefill_case(la, 3, 190, 5, dtype, 301, with_s0=True)
    assert eo <= tol(dtype) and es <= tol(dtype), (eo, es)


def test_prefill_tiny_f32_config(la):
    """Tiny fp32 prefill: batch 1, 8 heads, L = 1024, block 64, seed 1001; checked
    against the recurrence and against brute-force quadratic masked attention."""
    import torch

    w = workloads.TINY_F32
    q, k, v = workloads.qkv_host(w.seed, (1, w.seqlen, w.heads, 128), "f32")
    sl = workloads.slopes(w.heads)
    o, st = la.lt_prefill(to_device(q, "f32"), to_device(k, "f32"), to_device(v, "f32"),
                          torch.from_numpy(sl).cuda(), w.block)
    torch.cuda.synchronize()
    o_g, s_g = to_host_f32(o), to_host_f32(st)
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, sl)
    for h in range(w.heads):
        ob, sb = oracle.brute_force(q[0, :, h], k[0, :, h], v[0, :, h], sl[h])
        assert parity_err(o_ref[0, :, h], ob) < 1e-12
        assert parity_err(o_g[0, :, h], ob) <= TOL_F32
        assert parity_err(o_g[0, :, h], o_ref[0, :, h]) <= TOL_F32
        assert parity_err(s_g[0, h], sb) <= TOL_F32
        assert parity_err(s_g[0, h], s_ref[0, h]) <= TOL_F32


@pytest.mark.parametrize("block", [1, 16, 64, 100, 256, 4096])
def test_prefill_block_argument_does_not_change_value(la, block):
    eo, es = run_prefill_case(la, 1, 333, 2, "bf16", 401, block=block)
    assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)


def test_prefill_bf16_output(la):
    eo, es = run_prefill_case(la, 1, 257, 3, "bf16", 501, out_dtype="bf16")
    assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)


def test_prefill_extreme_slopes(la):
    """s = 0 (plain cumsum), tiny and huge slopes (decay underflows to exactly 0)."""
    import torch

    L, H = 300, 4
    q, k, v = workloads.qkv_host(601, (1, L, H, 128), "bf16")
    sl = np.array([0.0, 1e-6, 30.0, 500.0], np.float32)
    o, st = la.lt_prefill(to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"),
                          torch.from_numpy(sl).cuda(), 256)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, sl)
    o_g, s_g = to_host_f32(o), to_host_f32(st)
    assert np.isfinite(o_g).all() and np.isfinite(s_g).all()
    for h in range(H):
        assert parity_err(o_g[0, :, h], o_ref[0, :, h]) <= TOL_BF16, h
        assert parity_err(s_g[0, h], s_ref[0, h]) <= TOL_BF16, h


def test_prefill_state_in_place(la):
    """state_out == state_in updates the carried state in place."""
    import torch

    L, H = 150, 3
    q, k, v = workloads.qkv_host(701, (2, L, H, 128), "bf16")
    sl = workloads.slopes(H)
    s0 = workloads.state_host(702, (2, H, 128, 128))
    st = torch.from_numpy(s0).cuda()
    o, st2 = la.lt_prefill(to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"),
                           torch.from_numpy(sl).cuda(), 64, st, state_out=st)
    torch.cuda.synchronize()
    assert st2.data_ptr() == st.data_ptr()
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, sl, s0=s0)
    assert max_rel_states(to_host_f32(st), s_ref) <= TOL_BF16


def test_prefill_zero_length_passes_state_through(la):
    import torch

    H = 3
    s0 = workloads.state_host(801, (2, H, 128, 128))
    q = torch.empty((2, 0, H, 128), device="cuda", dtype=torch.bfloat16)
    sl = torch.from_numpy(workloads.slopes(H)).cuda()
    _, st = la.lt_prefill(q, q, q, sl, 256, torch.from_numpy(s0).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(to_host_f32(st), s0)
    _, st = la.lt_prefill(q, q, q, sl, 256)
    torch.cuda.synchronize()
    assert not to_host_f32(st).any()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_varlen_ragged_with_empty_sequences(la, dtype):
    import torch

    H = 4
    lens = [0, 1, 64, 65, 200, 0, 7, 130]
    cu = workloads.cu_seqlens(lens)
    T = int(cu[-1])
    print(f"[case] varlen lens={lens} dtype={dtype}", flush=True)
    q, k, v = workloads.qkv_host(901, (T, H, 128), dtype)
    sl = workloads.slopes(H)
    s0 = workloads.state_host(902, (len(lens), H, 128, 128))
    o, st = la.lt_prefill_varlen(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype),
                                 torch.from_numpy(cu).cuda(), torch.from_numpy(sl).cuda(), 256,
                                 torch.from_numpy(s0).cuda())
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence_packed(q, k, v, sl, cu, s0=s0)
    assert max_rel_per_head(to_host_f32(o), o_ref, cu) <= tol(dtype)
    assert max_rel_states(to_host_f32(st), s_ref) <= tol(dtype)


def test_chunked_prefill_equals_one_shot(la):
    """prefill(x[:a]) -> state -> prefill(x[a:], state) against the oracle over all of x."""
    import torch

    L, H, a = 777, 4, 321
    q, k, v = workloads.qkv_host(1101, (1, L, H, 128), "bf16")
    sl = workloads.slopes(H)
    dq, dk, dv = (to_device(x, "bf16") for x in (q, k, v))
    s_t = torch.from_numpy(sl).cuda()
    o1, st1 = la.lt_prefill(dq[:, :a].contiguous(), dk[:, :a].contiguous(),
                            dv[:, :a].contiguous(), s_t, 256)
    o2, st2 = la.lt_prefill(dq[:, a:].contiguous(), dk[:, a:].contiguous(),
                            dv[:, a:].contiguous(), s_t, 256, st1)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, sl)
    o_g = np.concatenate([to_host_f32(o1), to_host_f32(o2)], axis=1)
    cu = np.array([0, L])
    assert max_rel_per_head(o_g[0], o_ref[0], cu) <= TOL_BF16
    assert max_rel_states(to_host_f32(st2), s_ref) <= TOL_BF16


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_steps_continue_prefill(la, dtype):
    """prefill(L) then n decode steps against the oracle recurrence over L + n tokens."""
    import torch

    B, H, L, n = 3, 5, 100, 6
    q, k, v = workloads.qkv_host(1201, (B, L + n, H, 128), dtype)
    sl = workloads.slopes(H)
    s_t = torch.from_numpy(sl).cuda()
    dq, dk, dv = (to_device(x, dtype) for x in (q, k, v))
    _, st = la.lt_prefill(dq[:, :L].contiguous(), dk[:, :L].contiguous(),
                          dv[:, :L].contiguous(), s_t, 64)
    outs = []
    for t in range(L, L + n):
        outs.append(la.lt_decode(dq[:, t].contiguous(), dk[:, t].contiguous(),
                                 dv[:, t].contiguous(), s_t, st))
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, sl)
    for i, t in enumerate(range(L, L + n)):
        og = to_host_f32(outs[i])
        for b in range(B):
            for h in range(H):
                assert parity_err(og[b, h], o_ref[b, t, h]) <= tol(dtype), (t, b, h)
    assert max_rel_states(to_host_f32(st), s_ref) <= tol(dtype)


def test_decode_single_step_exact_inputs(la):
    """One decode step from a random fp32 state against the oracle's decode."""
    import torch

    B, H = 7, 6
    q, k, v = workloads.qkv_host(1301, (B, H, 128), "bf16")
    sl = workloads.slopes(H)
    s0 = workloads.state_host(1302, (B, H, 128, 128))
    st = torch.from_numpy(s0).cuda()
    o = la.lt_decode(to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"),
                     torch.from_numpy(sl).cuda(), st, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.decode(q, k, v, sl, s0)
    og, sg = to_host_f32(o), to_host_f32(st)
    for b in range(B):
        for h in range(H):
            assert parity_err(og[b, h], o_ref[b, h]) <= TOL_BF16
            # fp32 state update: a few ulps
            assert parity_err(sg[b, h], s_ref[b, h]) <= 1e-6


def test_prefill_is_deterministic(la):
    import torch

    q, k, v = workloads.qkv_host(1401, (1, 500, 8, 128), "bf16")
    sl = torch.from_numpy(workloads.slopes(8)).cuda()
    args = [to_device(x, "bf16") for x in (q, k, v)]
    o1, s1 = la.lt_prefill(*args, sl, 256)
    o2, s2 = la.lt_prefill(*args, sl, 256)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_launch_error_reports_status(la):
    """Argument errors surface as LightningError with the status code."""
    import torch

    q = torch.zeros((1, 8, 2, 64), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(la.LightningError) as e:
        la.lt_prefill(q, q, q, torch.zeros(2, device="cuda"), 64)
    assert e.value.status == la.LT_ERR_SHAPE


@pytest.mark.parametrize("L,H,with_s0", [(5000, 2, False), (9000, 1, True), (20000, 3, True),
                                         (16384, 4, False)])
def test_prefill_segmented_long_sequences(la, L, H, with_s0):
    """Few (sequence, head) pairs and long sequences take the segmented plan:
    a pre-pass over sequence pieces plus one workgroup per segment."""
    assert la.lt_prefill_workspace_bytes(1, L, H) > 0
    eo, es = run_prefill_case(la, 1, L, H, "bf16", 2000 + L, with_s0=with_s0)
    assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)


def test_prefill_segmented_matches_unsegmented(la):
    """The same inputs with and without a workspace (segmented vs one workgroup
    per sequence and head) both match the oracle."""
    import torch

    L, H = 12000, 2
    q, k, v = workloads.qkv_host(2101, (1, L, H, 128), "bf16")
    sl = workloads.slopes(H)
    s0 = workloads.state_host(2102, (1, H, 128, 128))
    args = [to_device(x, "bf16") for x in (q, k, v)]
    s_t = torch.from_numpy(sl).cuda()
    o_seg, st_seg = la.lt_prefill(*args, s_t, 256, torch.from_numpy(s0).cuda())
    o_one, st_one = la.lt_prefill(*args, s_t, 256, torch.from_numpy(s0).cuda(),
                                  workspace=torch.empty(0, device="cuda", dtype=torch.uint8))
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, sl, s0=s0)
    cu = np.array([0, L])
    for o_g, s_g in ((o_seg, st_seg), (o_one, st_one)):
        assert max_rel_per_head(to_host_f32(o_g)[0], o_ref[0], cu) <= TOL_BF16
        assert max_rel_states(to_host_f32(s_g), s_ref) <= TOL_BF16


def test_prefill_segmented_state_in_place(la):
    """Segmented plan with state_out == state_in: the pre-pass snapshots the
    carried-in state, so the in-place update cannot race."""
    import torch

    L, H = 10000, 2
    q, k, v = workloads.qkv_host(2201, (1, L, H, 128), "bf16")
    sl = workloads.slopes(H)
    s0 = workloads.state_host(2202, (1, H, 128, 128))
    st = torch.from_numpy(s0).cuda()
    la.lt_prefill(*(to_device(x, "bf16") for x in (q, k, v)), torch.from_numpy(sl).cuda(), 256,
                  st, state_out=st)
    torch.cuda.synchronize()
    _, s_ref = oracle.recurrence_batch(q, k, v, sl, s0=s0, want_o=False)
    assert max_rel_states(to_host_f32(st), s_ref) <= TOL_BF16


@pytest.mark.parametrize("batch,L,H,with_s0", [(1, 1, 64, True), (1, 65, 64, False),
                                               (1, 1000, 64, True), (2, 333, 40, True),
                                               (1, 200, 3, True)])
def test_prefill_value_slice_plan(la, batch, L, H, with_s0):
    """Short sequences with fewer than 256 (sequence, head) pairs take the
    value-slice kernel (4 workgroups of 32 value columns per head)."""
    assert la.lt_prefill_workspace_bytes(batch, L, H) == 0
    eo, es = run_prefill_case(la, batch, L, H, "bf16", 3000 + L + H, with_s0=with_s0)
    assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)


def test_prefill_value_slices_without_workspace(la):
    """A long sequence whose plan wants a workspace, called without one, falls
    back to value slices and still matches the oracle."""
    import torch

    L, H = 6000, 64
    assert la.lt_prefill_workspace_bytes(1, L, H) > 0
    q, k, v = workloads.qkv_host(3201, (1, L, H, 128), "bf16")
    sl = workloads.slopes(H)
    s0 = workloads.state_host(3202, (1, H, 128, 128))
    o, st = la.lt_prefill(*(to_device(x, "bf16") for x in (q, k, v)), torch.from_numpy(sl).cuda(),
                          256, torch.from_numpy(s0).cuda(),
                          workspace=torch.empty(0, device="cuda", dtype=torch.uint8))
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, sl, s0=s0)
    cu = np.array([0, L])
    assert max_rel_per_head(to_host_f32(o)[0], o_ref[0], cu) <= TOL_BF16
    assert max_rel_states(to_host_f32(st), s_ref) <= TOL_BF16


def test_prefill_value_slice_bf16_output_in_place(la):
    import torch

    L, H = 700, 64
    q, k, v = workloads.qkv_host(3101, (1, L, H, 128), "bf16")
    sl = workloads.slopes(H)
    s0 = workloads.state_host(3102, (1, H, 128, 128))
    st = torch.from_numpy(s0).cuda()
    o, _ = la.lt_prefill(*(to_device(x, "bf16") for x in (q, k, v)), torch.from_numpy(sl).cuda(),
                         256, st, state_out=st, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, sl, s0=s0)
    cu = np.array([0, L])
    assert max_rel_per_head(to_host_f32(o)[0], o_ref[0], cu) <= TOL_BF16
    assert max_rel_states(to_host_f32(st), s_ref) <= TOL_BF16


@pytest.mark.parametrize("B", [9, 37, 210])
def test_decode_batches_with_strided_order(la, B):
    """Decode visits sequences in a strided order for batch >= 8; every
    (sequence, head) output and state against the oracle."""
    import torch

    H = 3
    print(f"[case] decode B={B} H={H}", flush=True)
    q, k, v = workloads.qkv_host(1100 + B, (B, H, 128), "bf16")
    s0 = workloads.state_host(1200 + B, (B, H, 128, 128))
    sl = workloads.slopes(H)
    state = torch.from_numpy(s0).cuda()
    o = la.lt_decode(to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"),
                     torch.from_numpy(sl).cuda(), state)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.decode(q, k, v, sl, s0)
    og = to_host_f32(o)
    eo = max(parity_err(og[b, h], o_ref[b, h]) for b in range(B) for h in range(H))
    es = max_rel_states(to_host_f32(state), s_ref)
    assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_prefill_segmented_slope_mix(la, out_dtype):
    """Segmented plan (4 segments of 2,304 tokens) over heads whose decay sends
    them down both routes: heads with a short memory start every segment from
    zero and get the carried-in term added to their first tokens afterwards
    (slopes 0.02, 0.2, 1, 30: 831 corrected tokens down to none at all), heads
    with a long one (0, 1e-6, 0.005: 3,327 tokens, past the segment) take the
    pre-pass; with a carried-in state updated in place."""
    import torch

    L, H = 9000, 7
    sl = np.array([0.0, 1e-6, 0.005, 0.02, 0.2, 1.0, 30.0], np.float32)
    print(f"[case] segmented slope mix L={L} slopes={list(sl)} out={out_dtype}", flush=True)
    assert la.lt_prefill_workspace_bytes(1, L, H) > 0
    q, k, v = workloads.qkv_host(2301, (1, L, H, 128), "bf16")
    s0 = workloads.state_host(2302, (1, H, 128, 128))
    st = torch.from_numpy(s0).cuda()
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    o, _ = la.lt_prefill(*(to_device(x, "bf16") for x in (q, k, v)), torch.from_numpy(sl).cuda(), 256,
                         st, state_out=st, out_dtype=od)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, sl, s0=s0)
    o_g = to_host_f32(o)
    eo = max(parity_err(o_g[0, :, h], o_ref[0, :, h]) for h in range(H))
    es = max_rel_states(to_host_f32(st), s_ref)
    eb = max(segment_boundary_err(o_g[0, :, h], o_ref[0, :, h], 1, L, H, sl[h]) for h in range(H))
    print(f"[result] o {eo:.3e} state {es:.3e} segment-boundary rows {eb:.3e}", flush=True)
    assert eo <= TOL_BF16 and es <= TOL_BF16 and eb <= TOL_BF16, (eo, es, eb)


def test_prefill_segmented_warm_ranges_no_final_state(la):
    """Segmented plan over warm-up heads only, with no final state requested
    and a carried-in state (read by the ranges whose warm-up reaches the
    sequence start)."""
    import torch

    L, H = 9000, 4
    sl = np.array([0.02, 0.2, 1.0, 30.0], np.float32)
    print(f"[case] segmented warm ranges, no state_out, L={L} slopes={list(sl)}", flush=True)
    q, k, v = workloads.qkv_host(2311, (1, L, H, 128), "bf16")
    s0 = workloads.state_host(2312, (1, H, 128, 128))
    o, st = la.lt_prefill(*(to_device(x, "bf16") for x in (q, k, v)), torch.from_numpy(sl).cuda(), 256,
                          torch.from_numpy(s0).cuda(), want_state=False)
    torch.cuda.synchronize()
    assert st is None
    o_ref, _ = oracle.recurrence_batch(q, k, v, sl, s0=s0)
    og = to_host_f32(o)
    eo = max(parity_err(og[0, :, h], o_ref[0, :, h]) for h in range(H))
    print(f"[result] o {eo:.3e}", flush=True)
    assert eo <= TOL_BF16, eo


@pytest.mark.parametrize("L, H", [(16384, 64), (10240, 48), (9856, 32)])
def test_prefill_prepass_groups(la, L, H):
    """Many heads on the pre-pass (slopes scaled by 1e-4, so no head takes
    warm-up ranges): the kernels merge consecutive pre-pass pieces into groups
    (16384 tokens x 64 heads: 24 pieces of 512 in 4 groups of 6, every segment
    boundary inside a group; 10240 x 48: 16 pieces in groups of 3, the last of
    one piece, a group ending on the boundary at 6144; 9856 x 32: 15 pieces in
    groups of 2, one ending on the boundary at 5120, and a ragged last segment).
    Carried-in state updated in place; sampled heads against the oracle."""
    import torch

    sl = (workloads.slopes(H) * np.float32(1e-4)).astype(np.float32)
    print(f"[case] pre-pass groups L={L} H={H} slopes x1e-4", flush=True)
    q, k, v = workloads.qkv_host(2321 + L, (1, L, H, 128), "bf16")
    s0 = workloads.state_host(2322 + L, (1, H, 128, 128))
    st = torch.from_numpy(s0).cuda()
    o, _ = la.lt_prefill(*(to_device(x, "bf16") for x in (q, k, v)), torch.from_numpy(sl).cuda(), 256,
                         st, state_out=st)
    torch.cuda.synchronize()
    hs = [0, 1, 17, H - 9, H - 1]
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, sl, s0=s0, heads=hs)
    og = to_host_f32(o)[:, :, hs]
    eo = max(parity_err(og[0, :, i], o_ref[0, :, i]) for i in range(len(hs)))
    es = max_rel_states(to_host_f32(st)[:, hs], s_ref)
    print(f"[result] o {eo:.3e} state {es:.3e}", flush=True)
    assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)


def test_prefill_segmented_batch_slope_mix(la):
    """Segmented plan with several sequences (3 x 9000 tokens, 5 heads: 15
    pairs, 5 segments each) over heads on both routes (pre-pass: 0, 1e-6;
    warm-up ranges: 0.02, 0.3, 4), carried-in states, bf16 output."""
    import torch

    B, L, H = 3, 9000, 5
    sl = np.array([0.0, 1e-6, 0.02, 0.3, 4.0], np.float32)
    print(f"[case] segmented batch={B} L={L} slopes={list(sl)}", flush=True)
    assert la.lt_prefill_workspace_bytes(B, L, H) > 0
    q, k, v = workloads.qkv_host(2331, (B, L, H, 128), "bf16")
    s0 = workloads.state_host(2332, (B, H, 128, 128))
    o, st = la.lt_prefill(*(to_device(x, "bf16") for x in (q, k, v)), torch.from_numpy(sl).cuda(), 256,
                          torch.from_numpy(s0).cuda(), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, sl, s0=s0)
    og = to_host_f32(o)
    eo = max(parity_err(og[b, :, h], o_ref[b, :, h]) for b in range(B) for h in range(H))
    es = max_rel_states(to_host_f32(st), s_ref)
    print(f"[result] o {eo:.3e} state {es:.3e}", flush=True)
    assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)
