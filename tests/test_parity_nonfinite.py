"""GPU: NaN and Inf inputs against the fp64 oracle, on every prefill plan.

The contract (include/lightning.h): every output that the exact operator makes
non-finite is non-finite (NaN or Inf) on the GPU, whatever plan the call takes
(including warm-up ranges, which rebuild their carried-in state from a window
of earlier tokens and so cannot see a NaN or Inf from before it: a finishing
pass puts it back from the flagged end states of the earlier ranges; the
backward's reverse pass does the same with its carry, in mirrored token
order); every other output is
finite and within the parity bound, except outputs of earlier tokens of the
same 64-token block (counted from the sequence start) as a non-finite v: the
masked entries of the in-block product are zeros multiplied on the matrix
cores, and 0 * Inf is NaN there. These tests plant NaN and Inf in q, k, v and
the carried-in state of chosen (head, token) positions and check exactly that.
"""

import numpy as np
import pytest

import oracle
import workloads
from parity_util import TOL_BF16, ensure_built, parity_err, plan_segments, to_device, to_host_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def la():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    ensure_built()
    import linear_attention_amd

    return linear_attention_amd


def plant(q, k, v, spots):
    """spots: list of (tensor name, head, token, feature, value) in one sequence
    [L, H, d] (batch index 0). Returns the v spots (head, token, column) whose
    non-finite value may spread to earlier tokens of its 64-token block."""
    arrs = {"q": q, "k": k, "v": v}
    vspots = []
    for name, h, t, f, val in spots:
        arrs[name][0, t, h, f] = val
        if name == "v":
            vspots.append((h, t, f))
    return vspots


def allowed_mask(shape, vspots, whole_rows=False):
    """Entries the GPU may make NaN although the oracle keeps them finite: the
    earlier tokens of a non-finite v's 64-token block, in its column."""
    m = np.zeros(shape, bool)  # [L, H, d]
    for h, t, c in vspots:
        rows = slice(t // 64 * 64, t)
        if whole_rows:
            m[rows, h, :] = True
        else:
            m[rows, h, c] = True
    return m


def check(g, r, allowed, tol, what):
    """g (GPU), r (oracle): [L, H, d]. Non-finite masks and finite-row parity."""
    gbad, rbad = ~np.isfinite(g), ~np.isfinite(r)
    missed = rbad & ~gbad
    assert not missed.any(), f"{what}: finite on the GPU where the oracle is not: {np.argwhere(missed)[:4]}"
    extra = gbad & ~rbad & ~allowed
    assert not extra.any(), f"{what}: non-finite on the GPU where the oracle is finite: {np.argwhere(extra)[:4]}"
    worst = 0.0
    for h in range(r.shape[1]):
        rows = ~(gbad[:, h].any(-1) | rbad[:, h].any(-1))
        if rows.any():
            worst = max(worst, parity_err(g[rows, h], r[rows, h]))
    assert worst <= tol, f"{what}: finite rows parity {worst:.3e}"
    return int(rbad.sum()), int((gbad & ~rbad).sum()), worst


def check_states(g, r, what):
    """[H, d, d] final states: the same non-finite entries, finite ones in bound."""
    gbad, rbad = ~np.isfinite(g), ~np.isfinite(r)
    assert np.array_equal(gbad, rbad), f"{what}: state masks differ at {np.argwhere(gbad != rbad)[:4]}"
    worst = 0.0
    for h in range(r.shape[0]):
        rows = ~(gbad[h].any(-1) | rbad[h].any(-1))
        if rows.any():
            worst = max(worst, parity_err(g[h][rows], r[h][rows]))
    assert worst <= TOL_BF16, f"{what}: finite state rows {worst:.3e}"


# Slope mix of the segmented slope-mix test: heads 0-2 take the pre-pass (their
# memory outlasts a 2304-token segment), 3-6 warm-up ranges (warm-ups of 640,
# 128, 128 and 128 tokens; the ranges are about 2,250 tokens long).
MIX = np.array([0.0, 1e-6, 0.005, 0.02, 0.2, 1.0, 30.0], np.float32)
# (tensor, head, token, feature, value): segment 0 is [0, 2304), 1 [2304, 4608),
# 2 [4608, 6912), 3 [6912, 9000).
MIX_SPOTS = [
    ("k", 3, 1000, 5, np.nan),     # warm-up head: poisons the later ranges, whose warm-ups miss it
    ("v", 5, 1500, 17, np.inf),    # warm-up head, one value column, mid block
    ("k", 1, 700, 9, np.nan),      # pre-pass head
    ("v", 2, 2000, 3, -np.inf),    # pre-pass head, one column
    ("q", 6, 5000, 1, np.nan),     # one output row only
    ("k", 4, 4000, 0, -np.inf),    # warm-up head: poisons the later ranges
    ("q", 0, 8000, 2, np.inf),     # one output row only
]


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_nonfinite_segmented_both_routes(la, out_dtype):
    import torch

    L, H = 9000, 7
    assert plan_segments(1, L, H) == (4, 2304)
    print(f"[case] non-finite inputs, segmented L={L} slopes={list(MIX)} out={out_dtype}", flush=True)
    q, k, v = workloads.qkv_host(5101, (1, L, H, 128), "bf16")
    vspots = plant(q, k, v, MIX_SPOTS)
    s0 = workloads.state_host(5102, (1, H, 128, 128))
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    o, st = la.lt_prefill(*(to_device(x, "bf16") for x in (q, k, v)), torch.from_numpy(MIX).cuda(), 256,
                          torch.from_numpy(s0).cuda(), out_dtype=od)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, MIX, s0=s0)
    n_bad, n_extra, worst = check(to_host_f32(o)[0], o_ref[0], allowed_mask((L, H, 128), vspots),
                                  TOL_BF16, "o")
    check_states(to_host_f32(st)[0], s_ref[0], "state")
    print(f"[result] oracle non-finite {n_bad}, extra NaN on the GPU {n_extra}, finite rows {worst:.3e}",
          flush=True)
    assert n_bad > 100000  # the planted values reach most later outputs


def test_nonfinite_whole_head_and_value_slice_plans(la):
    """Unsegmented plans: value slices (few pairs, short sequences) and one
    workgroup per (sequence, head) (256 pairs), with a NaN in the carried-in
    state as well."""
    import torch

    for batch, L, H in ((1, 300, 4), (4, 200, 64)):
        print(f"[case] non-finite inputs, batch={batch} L={L} H={H}", flush=True)
        q, k, v = workloads.qkv_host(5200 + H, (batch, L, H, 128), "bf16")
        sl = workloads.slopes(H)
        spots = [("k", 0, 100, 3, np.nan), ("v", 1, 150, 7, np.inf), ("q", 2, 10, 0, np.nan)]
        vspots = plant(q, k, v, spots)
        s0 = workloads.state_host(5201 + H, (batch, H, 128, 128))
        s0[0, 3, 5, 5] = np.nan  # head 3: value column 5 of every output
        o, st = la.lt_prefill(*(to_device(x, "bf16") for x in (q, k, v)), torch.from_numpy(sl).cuda(), 256,
                              torch.from_numpy(s0).cuda())
        torch.cuda.synchronize()
        o_ref, s_ref = oracle.recurrence_batch(q, k, v, sl, s0=s0)
        og, sg = to_host_f32(o), to_host_f32(st)
        check(og[0], o_ref[0], allowed_mask((L, H, 128), vspots), TOL_BF16, f"o b0 {batch}x{L}x{H}")
        for b in range(1, batch):
            check(og[b], o_ref[b], np.zeros((L, H, 128), bool), TOL_BF16, f"o b{b}")
        for b in range(batch):
            check_states(sg[b], s_ref[b], f"state b{b}")


def test_nonfinite_fp32_inputs(la):
    """fp32 inputs (the fp32 kernel): the same contract at the fp32 bound."""
    import torch

    L, H = 200, 3
    q, k, v = workloads.qkv_host(5301, (1, L, H, 128), "f32")
    sl = workloads.slopes(H)
    vspots = plant(q, k, v, [("k", 0, 70, 3, np.nan), ("v", 1, 100, 7, np.inf), ("q", 2, 5, 0, np.nan)])
    o, st = la.lt_prefill(*(to_device(x, "f32") for x in (q, k, v)), torch.from_numpy(sl).cuda(), 64)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, sl)
    check(to_host_f32(o)[0], o_ref[0], allowed_mask((L, H, 128), vspots), 1e-5, "o fp32")
    check_states(to_host_f32(st)[0], s_ref[0], "state fp32")


def test_nonfinite_norm_gate_segmented(la):
    """The norm-gate epilogue on the segmented slope mix: the (token, head) rows
    of y that hold a NaN or Inf are exactly those whose sum o does (plus the
    documented v window), and the other rows match the oracle."""
    import torch

    L, H = 9000, 7
    print(f"[case] non-finite inputs, norm-gate segmented L={L}", flush=True)
    q, k, v = workloads.qkv_host(5401, (1, L, H, 128), "bf16")
    vspots = plant(q, k, v, MIX_SPOTS)
    gate = workloads.gate_host(5402, (1, L, H, 128))
    nw = workloads.norm_weight_host(5403, H)
    s0 = workloads.state_host(5404, (1, H, 128, 128))
    y, st = la.lt_prefill_norm_gate(*(to_device(x, "bf16") for x in (q, k, v)), torch.from_numpy(MIX).cuda(),
                                    to_device(gate, "bf16"), torch.from_numpy(nw).cuda(), workloads.NORM_EPS,
                                    256, torch.from_numpy(s0).cuda())
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence_batch(q, k, v, MIX, s0=s0)
    with np.errstate(invalid="ignore", over="ignore"):
        y_ref = oracle.norm_gate(o_ref, gate, nw, workloads.NORM_EPS)
    # Row level: the normalisation of a row whose sum holds an Inf is NaN in
    # that column and 0 elsewhere, of one holding a NaN NaN everywhere; which of
    # the two a non-finite element is can differ with the order of evaluation
    # (the block form's (q . k) v = +-Inf is the recurrence's sum of +-Inf
    # terms, NaN), so what must agree is which (token, head) rows hold one.
    yg = to_host_f32(y)[0]
    gbad = ~np.isfinite(yg).all(-1)
    rbad = ~np.isfinite(o_ref[0]).all(-1)
    allowed = allowed_mask((L, H, 128), vspots, whole_rows=True).any(-1)
    assert not (rbad & ~gbad).any(), f"finite y rows where the sum is not: {np.argwhere(rbad & ~gbad)[:4]}"
    assert not (gbad & ~rbad & ~allowed).any(), f"non-finite y rows: {np.argwhere(gbad & ~rbad & ~allowed)[:4]}"
    worst = max(parity_err(yg[~(gbad[:, h] | rbad[:, h]), h], y_ref[0][~(gbad[:, h] | rbad[:, h]), h])
                for h in range(H))
    assert worst <= TOL_BF16, worst
    check_states(to_host_f32(st)[0], s_ref[0], "state")
    print(f"[result] non-finite rows: oracle {int(rbad.sum())}, extra on the GPU {int((gbad & ~rbad).sum())}, "
          f"finite rows {worst:.3e}", flush=True)


def test_nonfinite_backward_segmented(la):
    """lt_prefill_backward on the segmented slope mix with a NaN in q near the
    end of the sequence (in the reverse pass's first ranges: the carry entries
    it reaches stay non-finite at every earlier token, past the warm-up windows
    of the later ranges, which the finishing pass covers from the records) and
    an Inf in dout."""
    import torch

    L, H = 9000, 7
    print(f"[case] non-finite inputs, backward segmented L={L}", flush=True)
    q, k, v = workloads.qkv_host(5501, (1, L, H, 128), "bf16")
    do = workloads.gate_host(5502, (1, L, H, 128))
    q[0, 8500, 4, 3] = np.nan        # warm-up head (s = 0.2), near the end of the sequence
    q[0, 8200, 1, 0] = np.nan        # pre-pass head
    do[0, 7000, 5, 9] = np.inf       # warm-up head (s = 1)
    ds = workloads.state_host(5503, (1, H, 128, 128))
    dq, dk, dv, dsi = la.lt_prefill_backward(*(to_device(x, "bf16") for x in (q, k, v, do)),
                                             torch.from_numpy(MIX).cuda(), 256, None,
                                             torch.from_numpy(ds).cuda())
    torch.cuda.synchronize()
    rq, rk, rv, rs = oracle.backward_batch(q, k, v, do, MIX, ds=ds)
    # in-block products of the reverse pass may spread a non-finite q or dout to
    # the other tokens of its 64-token block (blocks counted from the end), and
    # the dq pass (the forward operator on dout) spreads a non-finite dout like v
    bad_tokens = [(4, 8500), (1, 8200), (5, 7000)]
    allow = np.zeros((L, H, 128), bool)
    for h, t in bad_tokens:
        hi = L - (L - 1 - t) // 64 * 64
        allow[max(0, hi - 64):hi, h, :] = True
        allow[t // 64 * 64:t // 64 * 64 + 64, h, :] = True
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        n_bad, n_extra, worst = check(to_host_f32(g)[0], r[0], allow, TOL_BF16, name)
        print(f"[result] {name}: oracle non-finite {n_bad}, extra {n_extra}, finite rows {worst:.3e}", flush=True)
    check_states(to_host_f32(dsi)[0], rs[0], "d_state_in")


def test_nonfinite_decode(la):
    import torch

    B, H = 5, 4
    q, k, v = workloads.qkv_host(5601, (B, H, 128), "bf16")
    s0 = workloads.state_host(5602, (B, H, 128, 128))
    k[1, 2, 7] = np.nan
    v[3, 0, 9] = np.inf
    s0[4, 1, 2, 3] = np.nan
    sl = workloads.slopes(H)
    st = torch.from_numpy(s0).cuda()
    o = la.lt_decode(to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"),
                     torch.from_numpy(sl).cuda(), st)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.decode(q, k, v, sl, s0)
    og, sg = to_host_f32(o), to_host_f32(st)
    assert np.array_equal(~np.isfinite(og), ~np.isfinite(o_ref))
    assert np.array_equal(~np.isfinite(sg), ~np.isfinite(s_ref))
    fin = np.isfinite(o_ref).all(-1)
    assert max(parity_err(og[b, h], o_ref[b, h]) for b, h in zip(*np.nonzero(fin))) <= TOL_BF16
