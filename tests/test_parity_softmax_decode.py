"""GPU parity of lt_softmax_decode (one decode step of the softmax layer over a
KV cache) against oracle.softmax_decode: outputs (relative L2 per (sequence,
head) <= 1e-2), the appended cache rows (rope(k_new) within bf16 rounding,
v_new bit for bit), every other cache row untouched bit for bit, padding rows
zero; single-wave and split (flash-decoding) paths, and decode after a GPU
prefill against the prefill of one more token."""

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


def _inputs(seed, B, cap, Hq, Hkv):
    g = workloads.rng(seed)
    r = lambda *sh: workloads.round_bf16(g.standard_normal(sh, dtype=np.float32))
    return r(B, Hq, 128), r(B, Hkv, 128), r(B, Hkv, 128), r(B, cap, Hkv, 128), r(B, cap, Hkv, 128)


def _check(la, seed, B, cap, Hq, Hkv, lengths, R=64, out="f32", split=True, base=10000.0):
    import torch

    print(f"[case] softmax_decode seed={seed} B={B} cap={cap} Hq={Hq} Hkv={Hkv} lengths={list(lengths)} "
          f"R={R} out={out} split={split}", flush=True)
    q, kn, vn, kc, vc = _inputs(seed, B, cap, Hq, Hkv)
    kc_d, vc_d = to_device(kc, "bf16"), to_device(vc, "bf16")
    lens = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    od = torch.float32 if out == "f32" else torch.bfloat16
    ws = None if split else torch.empty(1, dtype=torch.uint8, device="cuda")
    o = la.lt_softmax_decode(to_device(q, "bf16"), to_device(kn, "bf16"), to_device(vn, "bf16"), kc_d, vc_d,
                             lens, rope_dims=R, rope_base=base, out_dtype=od, workspace=ws)
    torch.cuda.synchronize()
    o_ref, kc_ref, vc_ref = oracle.softmax_decode(q, kn, vn, kc, vc, np.array(lengths), rope_dims=R, base=base)
    og, kg, vg = to_host_f32(o), to_host_f32(kc_d), to_host_f32(vc_d)
    worst = 0.0
    for b, n in enumerate(lengths):
        if n < 0 or n >= cap:
            assert np.all(og[b] == 0), f"padding row {b} not zero"
            assert np.array_equal(kg[b], kc[b]) and np.array_equal(vg[b], vc[b]), f"padding row {b} touched the cache"
            continue
        worst = max(worst, max(parity_err(og[b, h], o_ref[b, h]) for h in range(Hq)))
        others = np.arange(cap) != n
        assert np.array_equal(kg[b, others], kc[b, others]) and np.array_equal(vg[b, others], vc[b, others])
        assert np.array_equal(vg[b, n], vn[b])
        assert parity_err(kg[b, n], kc_ref[b, n]) <= TOL_ROPE
    print(f"[result] o {worst:.3e}", flush=True)
    assert worst <= TOL_BF16, worst


@pytest.mark.parametrize("split", [True, False])
def test_softmax_decode_small(la, split):
    _check(la, 3001, 5, 300, 8, 2, [0, 17, 299, -1, 300], split=split)


def test_softmax_decode_many_splits(la):
    _check(la, 3002, 2, 4096, 16, 2, [4095, 1000])


def test_softmax_decode_group_of_32_bf16_out(la):
    _check(la, 3003, 3, 700, 32, 1, [699, 255, 256], out="bf16")


def test_softmax_decode_rope_variants(la):
    _check(la, 3004, 2, 520, 4, 4, [511, 33], R=0)
    _check(la, 3005, 2, 520, 8, 2, [100, 519], R=128, base=1e6)


def test_softmax_decode_after_prefill(la):
    """Prefill L tokens on the GPU, put its rope(k) and v in a cache, decode token L:
    equals row L of a GPU prefill of L + 1 tokens and the oracle's."""
    import torch

    B, L, Hq, Hkv, cap = 2, 333, 8, 2, 512
    q, k, v = workloads.softmax_qkv_host(3006, B, L + 1, Hq, Hkv)
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    print(f"[case] softmax decode after prefill B={B} L={L} cap={cap}", flush=True)
    _, kr = la.lt_softmax_prefill(qd[:, :L].contiguous(), kd[:, :L].contiguous(), vd[:, :L].contiguous())
    kc = torch.zeros((B, cap, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kc[:, :L] = kr
    vc[:, :L] = vd[:, :L]
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    o = la.lt_softmax_decode(qd[:, L].contiguous(), kd[:, L].contiguous(), vd[:, L].contiguous(), kc, vc, lens)
    o_full, kr_full = la.lt_softmax_prefill(qd, kd, vd)
    torch.cuda.synchronize()
    ref = oracle.softmax_attention(q, k, v)[:, L]
    og, of = to_host_f32(o), to_host_f32(o_full)[:, L]
    e1 = max(parity_err(og[b, h], ref[b, h]) for b in range(B) for h in range(Hq))
    e2 = max(parity_err(og[b, h], of[b, h]) for b in range(B) for h in range(Hq))
    print(f"[result] vs oracle {e1:.3e} vs prefill row {e2:.3e}", flush=True)
    assert e1 <= TOL_BF16 and e2 <= TOL_BF16
    assert torch.equal(kc[:, L], kr_full[:, L])  # same rope rows from both paths


def test_softmax_decode_m1_layer(la):
    """The softmax layer's decode workload: 16 sequences with 32768 cached tokens
    each (64 query heads, 8 K/V heads); sampled sequences against the oracle."""
    import torch

    wl = workloads.SOFTMAX_DECODE
    B, Hq, Hkv, ctx = wl.batch, wl.heads, wl.extra["kv_heads"], wl.extra["context"]
    cap = ctx + 1024
    print(f"[case] softmax_decode M1 layer B={B} ctx={ctx} cap={cap}", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed)
    rnd = lambda *sh: torch.randn(sh, generator=g, device="cuda").to(torch.bfloat16)
    q, kn, vn = rnd(B, Hq, 128), rnd(B, Hkv, 128), rnd(B, Hkv, 128)
    kc, vc = rnd(B, cap, Hkv, 128), rnd(B, cap, Hkv, 128)
    lengths = np.full(B, ctx, np.int64)
    lengths[3], lengths[7], lengths[11] = 1, 20000, cap - 1
    lens = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    sel = [0, 3, 7, 11, 15]
    kc0, vc0 = to_host_f32(kc[sel]), to_host_f32(vc[sel])
    o = la.lt_softmax_decode(q, kn, vn, kc, vc, lens, rope_dims=wl.extra["rope_dims"],
                             rope_base=wl.extra["rope_base"])
    torch.cuda.synchronize()
    ref, kref, _ = oracle.softmax_decode(to_host_f32(q)[sel], to_host_f32(kn)[sel], to_host_f32(vn)[sel], kc0, vc0,
                                         lengths[sel], rope_dims=wl.extra["rope_dims"], base=wl.extra["rope_base"])
    og = to_host_f32(o)[sel]
    worst = max(parity_err(og[i, h], ref[i, h]) for i in range(len(sel)) for h in range(Hq))
    kg = to_host_f32(kc[sel])
    wk = max(parity_err(kg[i, lengths[s]], kref[i, lengths[s]]) for i, s in enumerate(sel))
    print(f"[result] o {worst:.3e} appended k {wk:.3e}", flush=True)
    assert worst <= TOL_BF16 and wk <= TOL_ROPE
