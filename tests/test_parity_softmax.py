"""GPU parity of lt_softmax_prefill (causal softmax attention with grouped K/V
heads and partial RoPE, the hybrid's softmax layers) against
oracle.softmax_attention: every output at sizes spanning several 128-query
tiles and a ragged tail, sampled rows at the full 32768-token layer, and the
rope(k) rows it hands back. Relative L2 per (sequence, head) <= 1e-2 (bf16
inputs); rope(k) within bf16 rounding (relative L2 <= 5e-3)."""

import numpy as np
import pytest

import oracle
import workloads
from parity_util import TOL_BF16, ensure_built, parity_err, to_device, to_host_f32

pytestmark = pytest.mark.gpu

TOL_ROPE = 5e-3


@pytest.fixture(scope="module")
def la():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    ensure_built()
    import linear_attention_amd

    return linear_attention_amd


def _run(la, seed, B, L, Hq, Hkv, R, out, pos0=0, std=1.0, base=10000.0, scale=None):
    import torch

    print(f"[case] softmax_prefill seed={seed} B={B} L={L} Hq={Hq} Hkv={Hkv} R={R} out={out} "
          f"pos0={pos0} std={std}", flush=True)
    q, k, v = workloads.softmax_qkv_host(seed, B, L, Hq, Hkv, std=std)
    od = torch.float32 if out == "f32" else torch.bfloat16
    o, kr = la.lt_softmax_prefill(to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"),
                                  rope_dims=R, rope_base=base, scale=scale, pos0=pos0, out_dtype=od)
    torch.cuda.synchronize()
    o_ref = oracle.softmax_attention(q, k, v, rope_dims=R, base=base, scale=scale, pos0=pos0)
    kr_ref = oracle.rope(k, pos0 + np.arange(L), R, base)
    og, kg = to_host_f32(o), to_host_f32(kr)
    worst = max(parity_err(og[b, :, h], o_ref[b, :, h]) for b in range(B) for h in range(Hq))
    wk = max(parity_err(kg[b, :, g], kr_ref[b, :, g]) for b in range(B) for g in range(Hkv))
    print(f"[result] o {worst:.3e} k_rope {wk:.3e}", flush=True)
    assert worst <= TOL_BF16, worst
    assert wk <= TOL_ROPE, wk


@pytest.mark.parametrize("B,L,Hq,Hkv,R,out", [
    (2, 300, 8, 2, 64, "f32"),      # 3 query tiles, ragged tail of 44
    (1, 200, 4, 4, 0, "bf16"),      # no rotation, one K/V head per query head
    (1, 257, 8, 1, 128, "f32"),     # every feature rotated, one K/V head for all
    (1, 160, 4, 2, 32, "bf16"),
    (3, 129, 16, 2, 64, "f32"),     # one query past a tile
])
def test_softmax_prefill_small(la, B, L, Hq, Hkv, R, out):
    _run(la, 2000 + L + Hq, B, L, Hq, Hkv, R, out)


@pytest.mark.parametrize("L", [1, 2, 31, 63, 64, 65, 127, 128])
def test_softmax_prefill_short(la, L):
    _run(la, 2100 + L, 1, L, 4, 2, 64, "f32")


def test_softmax_prefill_far_positions(la):
    """Positions near 2^20 (angles of ~1e6 rad): the fp64 angle reduction."""
    _run(la, 2201, 1, 192, 4, 2, 64, "f32", pos0=(1 << 20) - 192)


def test_softmax_prefill_peaky_scores(la):
    """Scores of std ~9: the running maximum changes often and dominates."""
    _run(la, 2202, 1, 384, 4, 1, 64, "f32", std=3.0)


def test_softmax_prefill_base_and_scale(la):
    _run(la, 2203, 2, 140, 6, 3, 96, "f32", base=500000.0, scale=0.05)


def test_softmax_prefill_empty(la):
    import torch

    for B, L in ((0, 16), (1, 0)):
        q = torch.zeros((B, L, 8, 128), device="cuda", dtype=torch.bfloat16)
        k = torch.zeros((B, L, 2, 128), device="cuda", dtype=torch.bfloat16)
        o, kr = la.lt_softmax_prefill(q, k, k.clone())
        torch.cuda.synchronize()
        assert o.shape == (B, L, 8, 128) and kr.shape == k.shape


def test_softmax_prefill_m1_layer_sampled(la):
    """The full softmax layer: 32768 tokens, 64 query heads, 8 K/V heads, RoPE on
    64 dims; sampled query rows against the oracle's row form, all heads."""
    import torch

    wl = workloads.SOFTMAX_PREFILL
    B, L, Hq, Hkv = wl.batch, wl.seqlen, wl.heads, wl.extra["kv_heads"]
    R, base = wl.extra["rope_dims"], wl.extra["rope_base"]
    print(f"[case] softmax_prefill M1 layer B={B} L={L} Hq={Hq} Hkv={Hkv}", flush=True)
    q, k, v = workloads.softmax_qkv_device(wl.seed, B, L, Hq, Hkv)
    o, kr = la.lt_softmax_prefill(q, k, v, rope_dims=R, rope_base=base, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = [0, 1, 127, 128, 4095, 16383, 16384, 30001, 32766, 32767]
    qh, kh, vh = to_host_f32(q), to_host_f32(k), to_host_f32(v)
    ref = oracle.softmax_attention_rows(qh, kh, vh, rows, rope_dims=R, base=base)
    og = to_host_f32(o)[:, rows]
    worst = max(parity_err(og[0, i, h], ref[0, i, h]) for i in range(len(rows)) for h in range(Hq))
    kref = oracle.rope(kh[:, rows], np.array(rows), R, base)
    wk = max(parity_err(to_host_f32(kr)[0, rows][:, g], kref[0, :, g]) for g in range(Hkv))
    print(f"[result] o {worst:.3e} k_rope {wk:.3e}", flush=True)
    assert worst <= TOL_BF16 and wk <= TOL_ROPE


def test_softmax_prefill_moving_maximum(la):
    """Scores built so that the reference maximum moves many times: queries share
    a direction u (on the features RoPE leaves alone), the first 64 keys point
    against it (every query's first block has a strongly negative maximum,
    about -24 in log2 units) and later keys along it with a weight rising over
    the sequence (maxima up to about +36), so each query's maximum climbs by
    much more than the stale-maximum allowance in several steps."""
    import torch

    B, L, Hq, Hkv, R = 1, 1000, 8, 2, 64
    print(f"[case] softmax_prefill moving maximum L={L} Hq={Hq} Hkv={Hkv}", flush=True)
    g = workloads.rng(2204)
    u = np.zeros(128, np.float32)
    u[R:] = 1.0
    gam = np.where(np.arange(L) < 64, -2.0, -1.0 + 4.0 * np.arange(L) / L).astype(np.float32)
    q = workloads.round_bf16(g.standard_normal((B, L, Hq, 128), dtype=np.float32) + np.float32(1.5) * u)
    k = workloads.round_bf16(np.float32(0.5) * g.standard_normal((B, L, Hkv, 128), dtype=np.float32)
                             + gam[None, :, None, None] * u)
    v = workloads.round_bf16(g.standard_normal((B, L, Hkv, 128), dtype=np.float32))
    o, _ = la.lt_softmax_prefill(to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"),
                                 rope_dims=R, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref = oracle.softmax_attention(q, k, v, rope_dims=R)
    og = to_host_f32(o)
    worst = max(parity_err(og[0, :, h], o_ref[0, :, h]) for h in range(Hq))
    print(f"[result] o {worst:.3e}", flush=True)
    assert worst <= TOL_BF16, worst
