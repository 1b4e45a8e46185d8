"""GPU parity of lt_decode_slots (decode over a slot-indexed state pool)
against oracle.decode_slots: every output and every pool entry after several
steps; padding rows (ids < 0 or >= num_slots) give zero output and leave the
pool untouched, bit for bit. Relative L2 per (sequence, head) <= 1e-2 for bf16
inputs, <= 1e-5 for fp32."""

import numpy as np
import pytest

import oracle
import workloads
from parity_util import TOL_BF16, TOL_F32, ensure_built, parity_err, to_device, to_host_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def la():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    ensure_built()
    import linear_attention_amd

    return linear_attention_amd


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_slots_small_pool(la, dtype):
    import torch

    slots, H = 10, 3
    ids = np.array([3, -1, 7, 0, 9, 12], np.int32)
    B = len(ids)
    print(f"[case] decode_slots slots={slots} ids={list(ids)} dtype={dtype}", flush=True)
    pool0 = workloads.state_host(960, (slots, H, 128, 128))
    pool = torch.from_numpy(pool0).cuda()
    ids_d = torch.from_numpy(ids).cuda()
    sl = workloads.slopes(H)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    ref = pool0.astype(np.float64)
    worst = 0.0
    for t in range(4):
        q, k, v = workloads.qkv_host(970 + t, (B, H, 128), dtype)
        o = la.lt_decode_slots(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype),
                               torch.from_numpy(sl).cuda(), pool, ids_d)
        torch.cuda.synchronize()
        o_ref, ref = oracle.decode_slots(q, k, v, sl, ref, ids)
        og = to_host_f32(o)
        assert np.all(og[1] == 0.0) and np.all(og[5] == 0.0), "padding rows must be zero"
        worst = max(worst, max(parity_err(og[b, h], o_ref[b, h]) for b in (0, 2, 3, 4) for h in range(H)))
    pg = to_host_f32(pool)
    for s in (1, 2, 4, 5, 6, 8):  # never addressed
        assert np.array_equal(pg[s], pool0[s]), f"slot {s} changed"
    es = max(parity_err(pg[s, h], ref[s, h]) for s in (0, 3, 7, 9) for h in range(H))
    print(f"[result] o {worst:.3e} pool {es:.3e}", flush=True)
    assert worst <= tol and es <= tol


def test_decode_slots_full_batch(la):
    """256 sequences x 64 heads scattered over a 512-slot pool (8 padding rows),
    three steps; all outputs and all addressed slots of sampled sequences."""
    import torch

    B, H, slots = 256, 64, 512
    rng = np.random.Generator(np.random.PCG64(980))
    ids = rng.permutation(slots)[:B].astype(np.int32)
    ids[rng.choice(B, 8, replace=False)] = -1
    print(f"[case] decode_slots full B={B} H={H} slots={slots}", flush=True)
    pool = workloads.state_device(981, (slots, H, 128, 128), std=0.05)
    pool0_sampled = {}
    sample = [int(b) for b in rng.choice(B, 12, replace=False)]
    ids_d = torch.from_numpy(ids).cuda()
    sl = workloads.slopes(H)
    refs = {b: to_host_f32(pool[int(ids[b])]).astype(np.float64) for b in sample if ids[b] >= 0}
    untouched = [s for s in range(slots) if s not in set(ids.tolist())][:6]
    for s in untouched:
        pool0_sampled[s] = to_host_f32(pool[s])
    worst = 0.0
    for t in range(3):
        g = torch.Generator(device="cuda")
        g.manual_seed(990 + t)
        qkv = (torch.randn((3, B, H, 128), generator=g, device="cuda")
               .mul_(workloads.INPUT_SCALE).to(torch.bfloat16))
        o = la.lt_decode_slots(qkv[0], qkv[1], qkv[2], torch.from_numpy(sl).cuda(), pool, ids_d)
        torch.cuda.synchronize()
        og = to_host_f32(o)
        for b in sample:
            if ids[b] < 0:
                assert np.all(og[b] == 0.0)
                continue
            x = [to_host_f32(qkv[j, b:b + 1]) for j in range(3)]
            o_ref, st = oracle.decode(x[0], x[1], x[2], sl, refs[b][None])
            refs[b] = st[0]
            worst = max(worst, max(parity_err(og[b, h], o_ref[0, h]) for h in range(H)))
    es = max(parity_err(to_host_f32(pool[int(ids[b])])[h], refs[b][h]) for b in refs for h in range(H))
    for s in untouched:
        assert np.array_equal(to_host_f32(pool[s]), pool0_sampled[s])
    print(f"[result] o {worst:.3e} pool {es:.3e}", flush=True)
    assert worst <= TOL_BF16 and es <= TOL_BF16
