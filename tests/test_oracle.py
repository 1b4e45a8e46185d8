"""Pins for the fp64 oracle, against things other than itself (CPU only).

Every check here compares an oracle formulation with an independent fact:
the quadratic masked form (one block spanning the sequence), the block form at
many block sizes, closed forms for one-hot inputs, the s = 0 cumulative sum,
the s -> infinity limit, a pure state-decay case, invariants (chunking, decode
continuation, linearity, head permutation), and the state size the pages print.
A mutation test shows that plausible mistakes in a recurrence fail the pins.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SLOPES = [0.0, 2.0 ** -8, float(np.float32(2.0 ** (-1 / 8))), 5.0, 50.0]
TOL = 1e-12


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def rand_unit(seed, L, d, with_s0):
    g = np.random.Generator(np.random.PCG64(seed))
    q, k, v = (g.standard_normal((L, d)).astype(np.float32) for _ in range(3))
    s0 = g.standard_normal((d, d)) if with_s0 else None
    return q, k, v, s0


def c_rec(q, k, v, s, s0=None):
    return oracle.recurrence(q, k, v, s, s0=s0)


# --------------------------------------------------------------------------
# The pin suite, written against any single-unit recurrence function f.
# --------------------------------------------------------------------------

def pin_failures(f):
    """Names of the pins that f(q, k, v, s, s0) -> (o, S) fails."""
    bad = []
    d = 4
    # 1. quadratic masked form, with and without a carried-in state
    for s in (0.0, 2.0 ** -8, 0.917, 5.0):
        for with_s0 in (False, True):
            q, k, v, s0 = rand_unit(7, 23, d, with_s0)
            o, S = f(q, k, v, s, s0)
            ob, Sb = oracle.brute_force(q, k, v, s, s0)
            if rel(o, ob) > 1e-10 or rel(S, Sb) > 1e-10:
                bad.append(f"brute_force s={s} s0={with_s0}")
    # 2. one-hot closed form: q_i = e_a, k_j0 = e_a, v_j0 = e_b
    L, a, b = 11, 1, 2
    for s in (0.3, 1.7):
        for j0 in (1, 4, 11):
            q = np.zeros((L, d), np.float32)
            k = np.zeros((L, d), np.float32)
            v = np.zeros((L, d), np.float32)
            q[:, a] = 1.0
            k[j0 - 1, a] = 1.0
            v[j0 - 1, b] = 1.0
            o, S = f(q, k, v, s, None)
            sf = float(np.float32(s))
            want_o = np.zeros((L, d))
            for i in range(j0, L + 1):
                want_o[i - 1, b] = math.exp(-sf * (i - j0))
            want_S = np.zeros((d, d))
            want_S[a, b] = math.exp(-sf * (L - j0))
            if rel(o, want_o) > 1e-12 or rel(S, want_S) > 1e-12:
                bad.append(f"one_hot s={s} j0={j0}")
    # 3. s = 0: plain causal cumulative sum o_i = q_i sum_{j<=i} k_j^T v_j
    q, k, v, _ = rand_unit(11, 17, d, False)
    o, S = f(q, k, v, 0.0, None)
    cums = np.cumsum(np.einsum("lr,lc->lrc", k.astype(np.float64), v.astype(np.float64)), axis=0)
    want = np.einsum("lr,lrc->lc", q.astype(np.float64), cums)
    if rel(o, want) > 1e-12 or rel(S, cums[-1]) > 1e-12:
        bad.append("cumsum s=0")
    # 4. s large: only the diagonal survives, o_i = (q_i . k_i) v_i
    o, S = f(q, k, v, 200.0, None)
    want = np.sum(q.astype(np.float64) * k, axis=1)[:, None] * v
    if rel(o, want) > 1e-12:
        bad.append("diagonal s=200")
    # 5. pure state decay: k = v = 0, q = e_a -> o_i = e^{-s i} S0[a], S_L = e^{-s L} S0
    L = 9
    q = np.zeros((L, d), np.float32)
    q[:, a] = 1.0
    z = np.zeros((L, d), np.float32)
    s0 = np.random.Generator(np.random.PCG64(3)).standard_normal((d, d))
    s = 0.4
    sf = float(np.float32(s))
    o, S = f(q, z, z, s, s0)
    want_o = np.stack([math.exp(-sf * i) * s0[a] for i in range(1, L + 1)])
    if rel(o, want_o) > 1e-12 or rel(S, math.exp(-sf * L) * s0) > 1e-12:
        bad.append("state_decay")
    return bad


def test_c_recurrence_passes_pins():
    assert pin_failures(c_rec) == []


def test_numpy_loop_passes_pins():
    assert pin_failures(oracle.recurrence_loop) == []


@pytest.mark.parametrize("block", [1, 2, 3, 7, 16, 64])
def test_block_form_passes_pins(block):
    assert pin_failures(lambda q, k, v, s, s0: oracle.block_form(q, k, v, s, block, s0)) == []


# --------------------------------------------------------------------------
# Mutation test: plausible mistakes must fail at least one pin.
# --------------------------------------------------------------------------

def _mut_loop(q, k, v, s, s0, *, order="update_first", transpose=False, sign=-1.0,
              decay_s0=True, diag=True, qside="left"):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    L, d = q.shape
    lam = math.exp(sign * float(np.float32(s)))
    S = np.zeros((d, d)) if s0 is None else np.array(s0, np.float64)
    o = np.zeros((L, d))
    for i in range(L):
        if order == "read_first":
            o[i] = q[i] @ S
        kv = np.outer(v[i], k[i]) if transpose else np.outer(k[i], v[i])
        S = (lam * S if (decay_s0 or i > 0) else S) + kv
        if order == "update_first":
            o[i] = (q[i] @ S) if qside == "left" else (S @ q[i])
            if not diag:
                o[i] -= (q[i] @ k[i]) * v[i]
    return o, S


MUTANTS = {
    "output_before_update": dict(order="read_first"),
    "transposed_kv": dict(transpose=True),
    "growth_instead_of_decay": dict(sign=+1.0),
    "undecayed_carried_state": dict(decay_s0=False),
    "diagonal_dropped": dict(diag=False),
    "state_read_transposed": dict(qside="right"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_fail_pins(name):
    kw = MUTANTS[name]
    with np.errstate(all="ignore"):  # the growth mutant overflows on purpose
        assert pin_failures(lambda q, k, v, s, s0: _mut_loop(q, k, v, s, s0, **kw)), name


def test_unmutated_loop_passes_pins():
    assert pin_failures(lambda q, k, v, s, s0: _mut_loop(q, k, v, s, s0)) == []


def _mut_block(q, k, v, s, s0, block, mistake):
    """Copy of the block form with one planted mistake."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    L, d = q.shape
    s = float(np.float32(s))
    S = np.zeros((d, d)) if s0 is None else np.array(s0, np.float64)
    o = np.zeros((L, d))
    for t0 in range(0, L, block):
        m = min(block, L - t0)
        Qt, Kt, Vt = q[t0:t0 + m], k[t0:t0 + m], v[t0:t0 + m]
        i = np.arange(1, m + 1, dtype=np.float64)
        diff = i[:, None] - i[None, :]
        D = np.where(diff >= 0, np.exp(-s * np.maximum(diff, 0.0)), 0.0)
        dq = np.exp(-s * (i - 1 if mistake == "dq_zero_based" else i))
        mm = block if mistake == "full_block_for_short" else m
        dk = np.exp(-s * (mm - i))
        if mistake == "strict_mask":
            D = np.where(diff > 0, D, 0.0)
        o[t0:t0 + m] = ((Qt @ Kt.T) * D) @ Vt + (Qt * dq[:, None]) @ S
        S = np.exp(-s * mm) * S + (Kt * dk[:, None]).T @ Vt
    return o, S


@pytest.mark.parametrize("mistake", ["dq_zero_based", "full_block_for_short", "strict_mask"])
def test_block_mutants_fail_pins(mistake):
    # block 4 over lengths 23, 11, 17, 9 leaves short last blocks
    assert pin_failures(lambda q, k, v, s, s0: _mut_block(q, k, v, s, s0, 4, mistake))


# --------------------------------------------------------------------------
# Direct comparisons at the sizes the survey asks for.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("s", SLOPES)
@pytest.mark.parametrize("with_s0", [False, True])
@pytest.mark.parametrize("L,d", [(1, 3), (2, 8), (37, 8), (203, 16)])
def test_recurrence_vs_brute_force(s, with_s0, L, d):
    q, k, v, s0 = rand_unit(L * 100 + d, L, d, with_s0)
    o, S = c_rec(q, k, v, s, s0)
    ob, Sb = oracle.brute_force(q, k, v, s, s0)
    assert rel(o, ob) < TOL
    assert rel(S, Sb) < TOL


@pytest.mark.parametrize("s", SLOPES)
@pytest.mark.parametrize("block", [1, 2, 3, 7, 16, 64, 203, 512])
def test_block_size_invariance(s, block):
    q, k, v, s0 = rand_unit(5, 203, 8, True)
    o, S = c_rec(q, k, v, s, s0)
    ob, Sb = oracle.block_form(q, k, v, s, block, s0)
    assert rel(ob, o) < TOL
    assert rel(Sb, S) < TOL


def test_one_hot_at_block_edges():
    """Closed form with the key at the first/last slot of a block and in a short last block."""
    L, d, B, a, b = 70, 4, 16, 0, 3
    s = float(np.float32(0.25))
    for j0 in (1, 16, 17, 32, 64, 65, 70):
        q = np.zeros((L, d), np.float32)
        k = np.zeros((L, d), np.float32)
        v = np.zeros((L, d), np.float32)
        q[:, a] = 1.0
        k[j0 - 1, a] = 1.0
        v[j0 - 1, b] = 1.0
        want_o = np.zeros((L, d))
        for i in range(j0, L + 1):
            want_o[i - 1, b] = math.exp(-s * (i - j0))
        want_S = np.zeros((d, d))
        want_S[a, b] = math.exp(-s * (L - j0))
        for fn in (lambda: c_rec(q, k, v, s), lambda: oracle.block_form(q, k, v, s, B)):
            o, S = fn()
            assert rel(o, want_o) < 1e-13, j0
            assert rel(S, want_S) < 1e-13, j0


def test_chunk_invariance():
    q, k, v, s0 = rand_unit(9, 150, 8, True)
    s = 0.05
    o, S = c_rec(q, k, v, s, s0)
    for a in (1, 64, 149):
        o1, S1 = c_rec(q[:a], k[:a], v[:a], s, s0)
        o2, S2 = c_rec(q[a:], k[a:], v[a:], s, S1)
        assert rel(np.concatenate([o1, o2]), o) < TOL
        assert rel(S2, S) < TOL


def test_decode_continuation():
    """prefill(L) then n decode steps equals prefill(L + n)."""
    H, d, L, n = 3, 8, 40, 5
    g = np.random.Generator(np.random.PCG64(21))
    q, k, v = (g.standard_normal((1, L + n, H, d)).astype(np.float32) for _ in range(3))
    sl = workloads.slopes(H)
    o_full, S_full = oracle.recurrence_batch(q, k, v, sl)
    _, S = oracle.recurrence_batch(q[:, :L], k[:, :L], v[:, :L], sl)
    for t in range(L, L + n):
        o_t, S = oracle.decode(q[:, t], k[:, t], v[:, t], sl, S)
        assert rel(o_t, o_full[:, t]) < TOL
    assert rel(S, S_full) < TOL


def test_linearity_in_q_and_v():
    q1, k, v1, s0 = rand_unit(31, 60, 8, False)
    q2, _, v2, _ = rand_unit(32, 60, 8, False)
    s, al, be = 0.1, 0.7, -1.3  # (float64 combinations: NumPy keeps float32 * python float in float32)
    oq1, _ = oracle.recurrence_loop(q1, k, v1, s)
    oq2, _ = oracle.recurrence_loop(q2, k, v1, s)
    oq, _ = oracle.recurrence_loop(al * q1.astype(np.float64) + be * q2.astype(np.float64), k, v1, s)
    assert rel(oq, al * oq1 + be * oq2) < TOL
    ov2, S2 = oracle.recurrence_loop(q1, k, v2, s)
    ov, Sv = oracle.recurrence_loop(q1, k, al * v1.astype(np.float64) + be * v2.astype(np.float64), s)
    _, S1 = oracle.recurrence_loop(q1, k, v1, s)
    assert rel(ov, al * oq1 + be * ov2) < TOL
    assert rel(Sv, al * S1 + be * S2) < TOL


def test_heads_and_sequences_independent():
    """Permuting heads together with their slopes permutes the outputs; packing changes nothing."""
    H, d = 5, 8
    lens = [13, 1, 0, 40]
    cu = workloads.cu_seqlens(lens)
    T = int(cu[-1])
    g = np.random.Generator(np.random.PCG64(41))
    q, k, v = (g.standard_normal((T, H, d)).astype(np.float32) for _ in range(3))
    s0 = g.standard_normal((len(lens), H, d, d))
    sl = workloads.slopes(H)
    o, S = oracle.recurrence_packed(q, k, v, sl, cu, s0=s0)
    perm = [3, 0, 4, 1, 2]
    op, Sp = oracle.recurrence_packed(q[:, perm], k[:, perm], v[:, perm], sl[perm], cu,
                                      s0=s0[:, perm])
    assert rel(op, o[:, perm]) < TOL
    assert rel(Sp, S[:, perm]) < TOL
    for si, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        for h in range(H):
            ou, Su = oracle.recurrence_loop(q[a:b, h], k[a:b, h], v[a:b, h], sl[h], s0[si, h])
            assert rel(o[a:b, h], ou) < TOL
            assert rel(S[si, h], Su) < TOL
    # a zero-length sequence returns its carried-in state untouched
    assert np.array_equal(S[2], s0[2])


def test_heads_subset_matches_all():
    H, d, L = 6, 8, 33
    g = np.random.Generator(np.random.PCG64(51))
    q, k, v = (g.standard_normal((2, L, H, d)).astype(np.float32) for _ in range(3))
    sl = workloads.slopes(H)
    o, S = oracle.recurrence_batch(q, k, v, sl)
    o2, S2 = oracle.recurrence_batch(q, k, v, sl, heads=[4, 1])
    assert np.array_equal(o2, o[:, :, [4, 1]])
    assert np.array_equal(S2, S[:, [4, 1]])


def test_state_size_matches_pages():
    """The state the oracle carries (d x d per head) reproduces the sizes printed in §04."""
    gold = json.load(open(os.path.join(GOLDEN, "state_cache_sizes.json")))
    H, d = 64, 128
    q = np.zeros((1, 1, H, d), np.float32)
    _, S = oracle.recurrence_batch(q, q, q, workloads.slopes(H), want_o=False)
    per_layer_fp32 = S[0].size * 4
    assert S.shape == (1, H, d, d)
    p = gold["printed"]
    mb = gold["lightning_layers"] * per_layer_fp32 / 1e6
    assert round(mb, 2) == p["lightning_state_MB"]
    # softmax layers: K and V, 8 KV heads x 128, BF16, per token
    kv_per_layer_token = 2 * 8 * 128 * 2
    sm_gb = gold["softmax_layers"] * kv_per_layer_token * gold["context_tokens"] / 1e9
    all_gb = gold["all_layers"] * kv_per_layer_token * gold["context_tokens"] / 1e9
    assert round(sm_gb, 2) == p["softmax_kv_GB"]
    assert round(all_gb, 2) == p["all_gqa_kv_GB"]
    assert round(sm_gb + mb / 1e3, 2) == p["hybrid_total_GB"]
    assert round(100 * (1 - (sm_gb + mb / 1e3) / all_gb), 1) == p["saving_vs_all_gqa_percent"]


def test_workload_slopes_exact():
    """H = 8 slopes are 2^-1 .. 2^-8 exactly; H = 64 runs from 2^(-1/8) to 2^-8."""
    s8 = workloads.slopes(8)
    assert list(s8) == [2.0 ** -(h + 1) for h in range(8)]
    s64 = workloads.slopes(64)
    assert s64[-1] == 2.0 ** -8
    assert abs(s64[0] - 2.0 ** (-1 / 8)) < 1e-7


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1e-3], np.float32)
    r = workloads.round_bf16(x)
    assert r[0] == 1.0
    assert r[1] == 1.0            # tie -> even mantissa
    assert r[2] == 1.0 + 2 ** -6  # tie -> even (rounds up)
    assert r[3] == -2.5
    assert abs(r[4] - 1e-3) / 1e-3 < 2 ** -8
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)


# --------------------------------------------------------------------------
# Post-sum normalisation and gating (oracle.norm_gate)
# --------------------------------------------------------------------------

def _ng_inputs(seed, T=5, H=3, d=8):
    g = np.random.Generator(np.random.PCG64(seed))
    o = g.standard_normal((T, H, d)) * g.uniform(0.1, 10.0, (T, H, 1))
    gate = g.standard_normal((T, H, d))
    w = g.uniform(0.5, 2.0, (H, d))
    return o, gate, w


def norm_gate_pin_failures(f):
    """Names of the pins that f(o, gate, weight, eps) fails."""
    bad = []
    o, gate, w = _ng_inputs(11)
    T, H, d = o.shape
    ones = np.ones((H, d))
    big = np.full_like(gate, 40.0)  # sigmoid(40) rounds to 1 in fp64
    # 1. unit root mean square with weight 1, gate -> 1, eps = 0
    y = f(o, big, ones, 0.0)
    if np.max(np.abs(np.sqrt(np.mean(y * y, axis=-1)) - 1.0)) > 1e-12:
        bad.append("unit rms")
    # 2. with eps: rms(y) = sqrt(ms / (ms + eps))
    eps = 0.37
    ms = np.mean(o * o, axis=-1)
    y = f(o, big, ones, eps)
    if np.max(np.abs(np.sqrt(np.mean(y * y, axis=-1)) - np.sqrt(ms / (ms + eps)))) > 1e-12:
        bad.append("rms with eps")
    # 3. scale invariance and odd symmetry (eps = 0)
    y0 = f(o, gate, w, 0.0)
    if rel(f(3.7 * o, gate, w, 0.0), y0) > 1e-13 or rel(f(-o, gate, w, 0.0), -y0) > 1e-13:
        bad.append("scale invariance")
    # 4. one-hot closed form, every head with its own hot feature b_h:
    #    o_h = a e_{b_h} -> y_{h, b_h} = a / sqrt(a^2/d + eps) w[h, b_h] sigmoid(g_{h, b_h})
    a = 2.5
    oh = np.zeros((1, H, d))
    for hh in range(H):
        oh[0, hh, (3 + 2 * hh) % d] = a
    y = f(oh, gate[:1], w, eps)
    for hh in range(H):
        b = (3 + 2 * hh) % d
        want = a / math.sqrt(a * a / d + eps) * w[hh, b] / (1.0 + math.exp(-gate[0, hh, b]))
        others = np.delete(y[0, hh], b)
        if abs(y[0, hh, b] - want) > 1e-12 * abs(want) or np.max(np.abs(others)) > 0.0:
            bad.append(f"one-hot head {hh}")
    # 5. gate values with exact sigmoids: 0 -> 1/2, ln 3 -> 3/4
    yb = f(o, big, w, eps)
    if rel(f(o, np.zeros_like(gate), w, eps), 0.5 * yb) > 1e-13:
        bad.append("gate 0")
    if rel(f(o, np.full_like(gate, math.log(3.0)), w, eps), 0.75 * yb) > 1e-13:
        bad.append("gate ln 3")
    # 6. linear in the weight
    if rel(f(o, gate, 2.0 * w, eps), 2.0 * f(o, gate, w, eps)) > 1e-13:
        bad.append("weight linearity")
    # 7. heads are normalised independently
    o2 = o.copy()
    o2[:, 0] *= 100.0
    o2[:, 2] = np.random.Generator(np.random.PCG64(3)).standard_normal((T, d))
    if rel(f(o2, gate, w, eps)[:, 1], f(o, gate, w, eps)[:, 1]) > 1e-13:
        bad.append("per-head")
    # 8. feature permutation equivariance
    perm = np.random.Generator(np.random.PCG64(5)).permutation(d)
    if rel(f(o[..., perm], gate[..., perm], w[:, perm], eps), f(o, gate, w, eps)[..., perm]) > 1e-13:
        bad.append("permutation")
    return bad


def test_norm_gate_passes_pins():
    assert norm_gate_pin_failures(oracle.norm_gate) == []


def _ng_mutant(mistake):
    def f(o, gate, weight, eps):
        o = np.asarray(o, np.float64)
        g = np.asarray(gate, np.float64)
        w = np.asarray(weight, np.float64)
        x = o - o.mean(axis=-1, keepdims=True) if mistake == "layernorm" else o
        if mistake == "l2":
            den = np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
        elif mistake == "all_heads":
            den = np.sqrt(np.mean(x * x, axis=(-2, -1), keepdims=True) + eps)
        elif mistake == "no_eps":
            den = np.sqrt(np.mean(x * x, axis=-1, keepdims=True))
        elif mistake == "eps_outside":
            den = np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps
        else:
            den = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
        if mistake == "tanh":
            act = np.tanh(g)
        elif mistake == "gate_sign":
            act = 1.0 / (1.0 + np.exp(g))
        else:
            act = 1.0 / (1.0 + np.exp(-g))
        wt = w[::-1] if mistake == "weight_heads_reversed" else w
        return x / den * wt * act
    return f


@pytest.mark.parametrize("mistake", ["layernorm", "l2", "all_heads", "no_eps", "eps_outside",
                                     "tanh", "gate_sign", "weight_heads_reversed"])
def test_norm_gate_mutants_fail_pins(mistake):
    with np.errstate(all="ignore"):
        assert norm_gate_pin_failures(_ng_mutant(mistake)), mistake


def test_norm_gate_unmutated_mutant_passes():
    assert norm_gate_pin_failures(_ng_mutant(None)) == []


def test_norm_gate_of_decode_matches_prefill_rows():
    """The epilogue of a decode step equals the epilogue of the matching prefill row."""
    g = np.random.Generator(np.random.PCG64(21))
    L, H, d = 9, 2, 8
    q, k, v = (g.standard_normal((1, L, H, d)).astype(np.float32) for _ in range(3))
    sl = np.array([0.3, 0.01], np.float32)
    gate = g.standard_normal((L, H, d))
    w = g.uniform(0.5, 2.0, (H, d))
    o, _ = oracle.recurrence_batch(q, k, v, sl)
    y_pre = oracle.norm_gate(o[0], gate, w, 1e-6)
    st = np.zeros((1, H, d, d))
    for t in range(L):
        ot, st = oracle.decode(q[:, t], k[:, t], v[:, t], sl, st)
        assert rel(oracle.norm_gate(ot[0], gate[t], w, 1e-6), y_pre[t]) < 1e-12


# --------------------------------------------------------------------------
# Decode over a state pool (oracle.decode_slots)
# --------------------------------------------------------------------------

def _slot_inputs(seed, B=4, H=2, d=8, slots=6):
    g = np.random.Generator(np.random.PCG64(seed))
    q, k, v = (g.standard_normal((B, H, d)).astype(np.float32) for _ in range(3))
    pool = g.standard_normal((slots, H, d, d))
    sl = np.array([0.2, 0.01], np.float32)[:H]
    return q, k, v, sl, pool


def test_decode_slots_identity_equals_decode():
    q, k, v, sl, pool = _slot_inputs(31, slots=4)
    o, new = oracle.decode_slots(q, k, v, sl, pool, np.arange(4))
    o2, st2 = oracle.decode(q, k, v, sl, pool)
    assert rel(o, o2) < 1e-14 and rel(new, st2) < 1e-14


def test_decode_slots_padding_and_untouched_slots():
    q, k, v, sl, pool = _slot_inputs(32)
    ids = np.array([4, -1, 1, 6])           # -1 and 6 (= num_slots) are padding
    o, new = oracle.decode_slots(q, k, v, sl, pool, ids)
    assert np.all(o[1] == 0.0) and np.all(o[3] == 0.0)
    for s_ in (0, 2, 3, 5):                 # slots nobody addressed
        assert np.array_equal(new[s_], pool[s_])
    # the live rows: one step of the recurrence on their own slot (brute-force one-token form)
    for b, s_ in ((0, 4), (2, 1)):
        for h in range(q.shape[1]):
            S = (np.exp(-np.float64(sl[h])) * pool[s_, h]
                 + np.outer(k[b, h].astype(np.float64), v[b, h].astype(np.float64)))
            assert rel(new[s_, h], S) < 1e-13
            assert rel(o[b, h], q[b, h].astype(np.float64) @ S) < 1e-13


def test_decode_slots_relabelling_invariance():
    """Permuting the pool and the ids the same way permutes the result."""
    q, k, v, sl, pool = _slot_inputs(33)
    ids = np.array([5, 0, 3, 2])
    perm = np.random.Generator(np.random.PCG64(34)).permutation(pool.shape[0])
    inv = np.argsort(perm)
    o1, p1 = oracle.decode_slots(q, k, v, sl, pool, ids)
    o2, p2 = oracle.decode_slots(q, k, v, sl, pool[perm], inv[ids])
    assert rel(o1, o2) < 1e-14 and rel(p1, p2[inv]) < 1e-14


# --------------------------------------------------------------------------
# Backward (oracle.backward_*): gradients of l = sum dO . O + <dS, S_L>
# --------------------------------------------------------------------------

def c_bwd(q, k, v, do, s, s0=None, ds=None):
    """Single-unit adapter of oracle.backward_packed: [L, d] rows."""
    L, d = q.shape
    r = lambda x: np.asarray(x, np.float32).reshape(L, 1, d)
    rs = lambda x: None if x is None else np.asarray(x, np.float64).reshape(1, 1, d, d)
    dq, dk, dv, ds0 = oracle.backward_packed(r(q), r(k), r(v), r(do), np.array([s], np.float32),
                                             [0, L], s0=rs(s0), ds=rs(ds))
    return dq[:, 0], dk[:, 0], dv[:, 0], ds0[0, 0]


def _loss_bf(q, k, v, s, s0, do, ds):
    o, S = oracle.brute_force(q, k, v, s, s0)
    return float(np.sum(o * do) + (0.0 if ds is None else np.sum(S * ds)))


def backward_pin_failures(f):
    """Names of the pins that f(q, k, v, do, s, s0, ds) -> (dq, dk, dv, ds0) fails."""
    bad = []
    d, L = 4, 11
    g = np.random.Generator(np.random.PCG64(41))
    for s in (0.0, 0.3, 2.0):
        for with_state in (False, True):
            q, k, v, do = (g.standard_normal((L, d)).astype(np.float32).astype(np.float64)
                           for _ in range(4))
            s0 = g.standard_normal((d, d)) if with_state else None
            ds = g.standard_normal((d, d)) if with_state else None
            dq, dk, dv, ds0 = f(q, k, v, do, s, s0, ds)
            # 1. central finite differences of the fp64 quadratic form, one input at a time
            eps = 1e-6
            base_s0 = s0 if s0 is not None else np.zeros((d, d))
            for name, grad in (("q", dq), ("k", dk), ("v", dv), ("s0", ds0)):
                delta = g.standard_normal(grad.shape)
                args = dict(q=q, k=k, v=v, s0=base_s0)
                plus, minus = dict(args), dict(args)
                plus[name] = args[name] + eps * delta
                minus[name] = args[name] - eps * delta
                fd = (_loss_bf(plus["q"], plus["k"], plus["v"], s, plus["s0"], do, ds)
                      - _loss_bf(minus["q"], minus["k"], minus["v"], s, minus["s0"], do, ds)) / (2 * eps)
                an = float(np.sum(grad * delta))
                if abs(fd - an) > 1e-6 * max(1.0, abs(fd)):
                    bad.append(f"finite difference d{name} s={s} state={with_state}")
            # 2. closed forms from the quadratic masked form
            sf = np.float64(np.float32(s))
            pos = np.arange(1, L + 1, dtype=np.float64)
            diff = pos[:, None] - pos[None, :]
            M = np.where(diff >= 0, np.exp(-sf * np.maximum(diff, 0.0)), 0.0)
            lq, lk = np.exp(-sf * pos), np.exp(-sf * (L - pos))
            S0 = base_s0
            dS = ds if ds is not None else np.zeros((d, d))
            dq_w = ((do @ v.T) * M) @ k + lq[:, None] * (do @ S0.T)
            dk_w = ((do @ v.T) * M).T @ q + lk[:, None] * (v @ dS.T)
            dv_w = ((q @ k.T) * M).T @ do + lk[:, None] * (k @ dS)
            ds0_w = (q * lq[:, None]).T @ do + np.exp(-sf * L) * dS
            for name, a, b in (("dq", dq, dq_w), ("dk", dk, dk_w), ("dv", dv, dv_w),
                               ("ds0", ds0, ds0_w)):
                if rel(a, b) > 1e-10:
                    bad.append(f"closed form {name} s={s} state={with_state}")
    # 3. s = 200: only the diagonal (and the final-state term of the last token) survives
    q, k, v, do = (g.standard_normal((L, d)) for _ in range(4))
    q, k, v, do = (x.astype(np.float32).astype(np.float64) for x in (q, k, v, do))
    dS = g.standard_normal((d, d))
    dq, dk, dv, ds0 = f(q, k, v, do, 200.0, None, dS)
    dots = np.sum(do * v, axis=1)
    dk_w = dots[:, None] * q
    dk_w[-1] += dS @ v[-1]
    dv_w = np.sum(q * k, axis=1)[:, None] * do
    dv_w[-1] += k[-1] @ dS
    if (rel(dq, dots[:, None] * k) > 1e-12 or rel(dk, dk_w) > 1e-12 or rel(dv, dv_w) > 1e-12
            or np.max(np.abs(ds0)) > 1e-80):
        bad.append("s=200 diagonal")
    # 4. linear in dO (eighths, so that dO1 + dO2 is exact in float32 too)
    do1 = g.integers(-16, 17, (L, d)) / 8.0
    do2 = g.integers(-16, 17, (L, d)) / 8.0
    r1, r2, r12 = (f(q, k, v, x, 0.3, None, None) for x in (do1, do2, do1 + do2))
    if any(rel(c, a + b) > 1e-12 for a, b, c in zip(r1, r2, r12)):
        bad.append("linear in dO")
    return bad


def test_backward_passes_pins():
    assert backward_pin_failures(c_bwd) == []


def _bwd_loop(q, k, v, do, s, s0=None, ds=None, mistake=None):
    """Per-token reverse-mode loop with switchable mistakes (mutation tests)."""
    L, d = q.shape
    lam = np.exp(-np.float64(np.float32(s)))
    S = np.zeros((d, d)) if s0 is None else np.array(s0, np.float64)
    dq = np.zeros((L, d))
    for t in range(L):
        prev = S.copy()
        S = lam * S + np.outer(k[t], v[t])
        dq[t] = (prev if mistake == "dq_prev_state" else S) @ do[t]
    R = np.zeros((d, d)) if (ds is None or mistake == "ds_ignored") else np.array(ds, np.float64)
    dk, dv = np.zeros((L, d)), np.zeros((L, d))
    for t in range(L - 1, -1, -1):
        G = np.outer(q[t], do[t]) + R
        dk[t] = (G.T if mistake == "dk_transposed" else G) @ v[t]
        dv[t] = G.T @ (q[t] if mistake == "dv_from_q" else k[t])
        R = G if mistake == "no_decay_carry" else lam * G
    ds0 = R / lam if mistake == "ds0_undecayed" else R
    return dq, dk, dv, ds0


def test_backward_numpy_loop_passes_pins():
    assert backward_pin_failures(_bwd_loop) == []


@pytest.mark.parametrize("mistake", ["dq_prev_state", "ds_ignored", "dk_transposed", "dv_from_q",
                                     "no_decay_carry", "ds0_undecayed"])
def test_backward_mutants_fail_pins(mistake):
    f = lambda q, k, v, do, s, s0, ds: _bwd_loop(q, k, v, do, s, s0, ds, mistake=mistake)
    with np.errstate(all="ignore"):
        assert backward_pin_failures(f), mistake


def test_backward_batch_matches_units():
    """Packed and batched entry points agree with the single-unit one."""
    g = np.random.Generator(np.random.PCG64(43))
    B, L, H, d = 2, 9, 3, 4
    q, k, v, do = (g.standard_normal((B, L, H, d)).astype(np.float32) for _ in range(4))
    sl = np.array([0.5, 0.05, 0.0], np.float32)
    s0 = g.standard_normal((B, H, d, d))
    ds = g.standard_normal((B, H, d, d))
    dq, dk, dv, ds0 = oracle.backward_batch(q, k, v, do, sl, s0=s0, ds=ds)
    for b in range(B):
        for h in range(H):
            r = c_bwd(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], float(sl[h]), s0[b, h], ds[b, h])
            for got, want in zip((dq[b, :, h], dk[b, :, h], dv[b, :, h], ds0[b, h]), r):
                assert rel(got, want) < 1e-14


# --------------------------------------------------------------------------
# Softmax GQA attention with partial RoPE (oracle.rope / softmax_attention /
# softmax_decode)
# --------------------------------------------------------------------------

def rope_pin_failures(f):
    """Pins of a rope(x, positions, rope_dims, base) function."""
    bad = []
    g = np.random.Generator(np.random.PCG64(51))
    d, R = 8, 4
    # explicit rotation: position 1, pair m = 0 (theta = 1), pair m = 1 (theta = base^-1/2)
    x = g.standard_normal((1, 1, d))
    y = f(x, [1], R, 100.0)
    for m, th in ((0, 1.0), (1, 100.0 ** -0.5)):
        a, b = x[0, 0, m], x[0, 0, m + R // 2]
        want = (a * math.cos(th) - b * math.sin(th), a * math.sin(th) + b * math.cos(th))
        if abs(y[0, 0, m] - want[0]) > 1e-12 or abs(y[0, 0, m + R // 2] - want[1]) > 1e-12:
            bad.append(f"rotation pair {m}")
    if not np.array_equal(y[0, 0, R:], x[0, 0, R:]):
        bad.append("unrotated features changed")
    # norm of every rotated pair preserved; rope_dims = 0 is the identity
    xs = g.standard_normal((7, 3, d))
    ys = f(xs, np.arange(7) * 13 + 5, R, 10000.0)
    for m in range(R // 2):
        if np.max(np.abs(np.hypot(ys[..., m], ys[..., m + R // 2]) - np.hypot(xs[..., m], xs[..., m + R // 2]))) > 1e-12:
            bad.append("pair norm")
    if not np.array_equal(f(xs, np.arange(7), 0, 10000.0), xs):
        bad.append("rope_dims 0")
    # relative position: rope(q, p1) . rope(k, p2) depends on p1 - p2 only
    q1, k1 = g.standard_normal((1, 1, d)), g.standard_normal((1, 1, d))
    dots = [float(np.sum(f(q1, [p + 9], R, 10000.0) * f(k1, [p], R, 10000.0))) for p in (0, 5, 1234)]
    if max(dots) - min(dots) > 1e-10:
        bad.append("relative position")
    return bad


def test_rope_passes_pins():
    assert rope_pin_failures(oracle.rope) == []


def _rope_interleaved(x, positions, rope_dims, base):
    x = np.asarray(x, np.float64)
    out = x.copy()
    half = rope_dims // 2
    th = np.float64(base) ** (-2.0 * np.arange(half) / rope_dims)
    ang = np.asarray(positions, np.float64)[:, None] * th[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., 0:rope_dims:2], x[..., 1:rope_dims:2]
    out[..., 0:rope_dims:2] = a * c - b * s
    out[..., 1:rope_dims:2] = a * s + b * c
    return out


def _rope_last_half(x, positions, rope_dims, base):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    y = oracle.rope(x[..., ::-1], positions, rope_dims, base)  # rotates the last features
    return y[..., ::-1]


@pytest.mark.parametrize("mutant", [_rope_interleaved, _rope_last_half])
def test_rope_mutants_fail_pins(mutant):
    assert rope_pin_failures(mutant)


def softmax_pin_failures(f):
    """Pins of f(q, k, v, rope_dims, base, scale, pos0) -> o (causal GQA attention)."""
    import torch

    bad = []
    g = np.random.Generator(np.random.PCG64(52))
    B, L, Hq, Hkv, d, R = 2, 13, 4, 2, 8, 4
    q, k, v = g.standard_normal((B, L, Hq, d)), g.standard_normal((B, L, Hkv, d)), g.standard_normal((B, L, Hkv, d))
    # 1. torch's scaled_dot_product_attention (fp64, CPU) on pre-rotated inputs
    for pos0, scale in ((0, None), (7, 0.3)):
        o = f(q, k, v, R, 10000.0, scale, pos0)
        pos = pos0 + np.arange(L)
        qr, kr = oracle.rope(q, pos, R, 10000.0), oracle.rope(k, pos, R, 10000.0)
        tq = torch.from_numpy(qr).permute(0, 2, 1, 3)
        tk = torch.from_numpy(kr).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
        tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=True, scale=(1 / math.sqrt(d) if scale is None else scale))
        if not (rel(o, ref.permute(0, 2, 1, 3).numpy()) <= 1e-12):
            bad.append(f"sdpa pos0={pos0}")
    # 2. q = 0: uniform weights, o_t = mean(v_0..v_t)
    o = f(np.zeros_like(q), k, v, R, 10000.0, None, 0)
    want = np.cumsum(v, axis=1) / np.arange(1, L + 1)[None, :, None, None]
    if not (rel(o[:, :, ::Hq // Hkv], want) <= 1e-12) or not (rel(o[:, :, 1::Hq // Hkv], want) <= 1e-12):
        bad.append("uniform")
    # 3. one token: o = v_0 of the head's group
    o = f(q[:, :1], k[:, :1], v[:, :1], R, 10000.0, None, 3)
    if not (rel(o, np.repeat(v[:, :1], Hq // Hkv, axis=2)) <= 1e-12):
        bad.append("single key")
    # 4. absolute shift invariance (RoPE is relative)
    if not (rel(f(q, k, v, R, 10000.0, None, 0), f(q, k, v, R, 10000.0, None, 1000)) <= 1e-10):
        bad.append("shift invariance")
    # 5. grouped heads: equal queries in one group give equal outputs; another
    #    group's K/V do not matter
    q2 = q.copy()
    q2[:, :, 1] = q2[:, :, 0]
    o = f(q2, k, v, R, 10000.0, None, 0)
    k3 = k.copy()
    k3[:, :, 1] += 5.0
    o3 = f(q2, k3, v, R, 10000.0, None, 0)
    if not (rel(o[:, :, 1], o[:, :, 0]) <= 1e-14) or not (rel(o3[:, :, :2], o[:, :, :2]) <= 1e-14):
        bad.append("grouped heads")
    return bad


def _sm(q, k, v, R, base, scale, pos0):
    return oracle.softmax_attention(q, k, v, rope_dims=R, base=base, scale=scale, pos0=pos0)


def test_softmax_attention_passes_pins():
    assert softmax_pin_failures(_sm) == []


def _sm_mutant(mistake):
    def f(q, k, v, R, base, scale, pos0):
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        B, L, Hq, d = q.shape
        Hkv = k.shape[2]
        sc = 1.0 / np.sqrt(d) if scale is None else scale
        if mistake == "no_scale":
            sc = 1.0
        pos = pos0 + np.arange(L)
        qr, kr = oracle.rope(q, pos, R, base), oracle.rope(k, pos, R, base)
        if mistake == "rope_q_only":
            kr = k
        mask = np.tril(np.ones((L, L), bool), k=-1 if mistake == "strict_mask" else 0)
        o = np.zeros((B, L, Hq, d))
        for b in range(B):
            for h in range(Hq):
                gh = h % Hkv if mistake == "head_modulo" else h // (Hq // Hkv)
                s = sc * (qr[b, :, h] @ kr[b, :, gh].T)
                s = np.where(mask, s, -np.inf)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                o[b, :, h] = (p / p.sum(axis=1, keepdims=True)) @ v[b, :, gh]
        return o
    return f


@pytest.mark.parametrize("mistake", ["no_scale", "strict_mask", "head_modulo", "rope_q_only"])
def test_softmax_mutants_fail_pins(mistake):
    with np.errstate(all="ignore"):
        assert softmax_pin_failures(_sm_mutant(mistake)), mistake


def test_softmax_unmutated_mutant_passes():
    assert softmax_pin_failures(_sm_mutant(None)) == []


def test_softmax_decode_matches_last_prefill_row():
    """Decode over a cache of the first n tokens (rope applied) equals row n of the
    prefill; the cache gains the new entries; padding rows stay zero."""
    g = np.random.Generator(np.random.PCG64(53))
    B, L, Hq, Hkv, d, R, cap = 3, 10, 4, 2, 8, 4, 16
    q, k, v = g.standard_normal((B, L, Hq, d)), g.standard_normal((B, L, Hkv, d)), g.standard_normal((B, L, Hkv, d))
    o_full = oracle.softmax_attention(q, k, v, rope_dims=R)
    n = L - 1
    kc = np.zeros((B, cap, Hkv, d))
    vc = np.zeros((B, cap, Hkv, d))
    kc[:, :n] = oracle.rope(k[:, :n], np.arange(n), R, 10000.0)
    vc[:, :n] = v[:, :n]
    lengths = np.array([n, n, cap])  # the last row is padding (length == capacity)
    o, kc2, vc2 = oracle.softmax_decode(q[:, n], k[:, n], v[:, n], kc, vc, lengths, rope_dims=R)
    assert rel(o[:2], o_full[:2, n]) < 1e-12
    assert np.all(o[2] == 0) and np.array_equal(kc2[2], kc[2]) and np.array_equal(vc2[2], vc[2])
    assert rel(kc2[:2, n], oracle.rope(k[:2, n][:, None], [n], R, 10000.0)[:, 0]) < 1e-14


def test_softmax_rows_match_full_form():
    """The row-sampled form agrees with the full form at every sampled row (first,
    last, a middle row, a repeated row), with a position offset and GQA groups."""
    g = np.random.Generator(np.random.PCG64(59))
    B, L, Hq, Hkv, d, R = 2, 11, 6, 2, 8, 4
    q, k, v = g.standard_normal((B, L, Hq, d)), g.standard_normal((B, L, Hkv, d)), g.standard_normal((B, L, Hkv, d))
    rows = [0, 5, 10, 5]
    full = oracle.softmax_attention(q, k, v, rope_dims=R, base=500.0, scale=0.3, pos0=77)
    part = oracle.softmax_attention_rows(q, k, v, rows, rope_dims=R, base=500.0, scale=0.3, pos0=77)
    assert rel(part, full[:, rows]) < 1e-13


def test_recurrence_propagates_non_finite_inputs():
    """The exact operator's non-finite pattern (reading 14: NaN and Inf
    propagate), pinned by what the recurrence S <- e^{-s} S + k^T v, o = q S
    implies: a NaN in feature r of k_j makes row r of every later state NaN, so
    every output from token j on is NaN and every earlier one finite; an Inf in
    column c of v_j makes column c of every later state infinite, so column c of
    every output from token j on is non-finite and nothing else is; a NaN in q_i
    touches output i only; a NaN at (r, c) of S_0 column c of every output."""
    L, d, s = 40, 16, 0.3
    g = np.random.default_rng(77)
    base = [g.standard_normal((L, d)).astype(np.float32) for _ in range(3)]

    def run(q=None, k=None, v=None, s0=None):
        x = [b.copy() for b in base]
        for i, (arr, spot) in enumerate(((x[0], q), (x[1], k), (x[2], v))):
            if spot:
                arr[spot[0], spot[1]] = spot[2]
        o, S = oracle.recurrence(x[0], x[1], x[2], s, s0=s0)
        return ~np.isfinite(o), ~np.isfinite(S)

    bad, sbad = run(k=(10, 3, np.nan))
    assert not bad[:10].any() and bad[10:].all()
    assert sbad[3].all() and not np.delete(sbad, 3, axis=0).any()
    bad, sbad = run(v=(25, 5, np.inf))
    assert not bad[:25].any() and bad[25:, 5].all() and not np.delete(bad, 5, axis=1).any()
    assert sbad[:, 5].all() and not np.delete(sbad, 5, axis=1).any()
    bad, _ = run(q=(7, 0, np.nan))
    assert bad[7].all() and not np.delete(bad, 7, axis=0).any()
    s0 = np.zeros((d, d))
    s0[2, 9] = np.nan
    bad, sbad = run(s0=s0)
    assert bad[:, 9].all() and not np.delete(bad, 9, axis=1).any()
    assert sbad[2, 9] and sbad.sum() == 1
