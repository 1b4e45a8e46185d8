"""CPU checks of the Python binding's argument validation (no GPU needed).

The C ABI receives only pointers and sizes, so a tensor of the wrong shape or
dtype would be read or written out of bounds on the device. The torch wrappers
check the shape, dtype and layout of every tensor argument first, and only then
its device, so each mismatch below raises an error naming the argument on CPU
tensors too, before anything reaches the library.
"""

import pytest

torch = pytest.importorskip("torch")

from parity_util import ensure_built  # noqa: E402

ensure_built()

import linear_attention_amd as la  # noqa: E402

BF, F32 = torch.bfloat16, torch.float32
B, L, H, D = 2, 8, 3, 128


def z(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


def raises(fn, exc, name):
    with pytest.raises(exc) as e:
        fn()
    assert name in str(e.value), str(e.value)


def qkv4():
    return z(B, L, H, D), z(B, L, H, D), z(B, L, H, D)


def test_all_checks_pass_up_to_the_device_check():
    """Well-formed CPU arguments get as far as the device check."""
    raises(lambda: la.lt_prefill(*qkv4(), z(H, dtype=F32), 64), ValueError, "device tensor")


@pytest.mark.parametrize("kw,exc,name", [
    (dict(slopes=z(H)), TypeError, "slopes"),                        # bf16 slopes
    (dict(slopes=z(H, dtype=torch.float64)), TypeError, "slopes"),  # would be read as fp32
    (dict(slopes=z(H + 1, dtype=F32)), ValueError, "slopes"),
    (dict(o=z(B, L - 1, H, D, dtype=F32)), ValueError, "o"),          # too small an output
    (dict(o=z(B, L, H, D, dtype=torch.int32)), TypeError, "o"),
    (dict(o=z(B, L, H, D, dtype=F32), out_dtype=BF), TypeError, "o"),
    (dict(state_in=z(B, H, D, D)), TypeError, "state_in"),
    (dict(state_in=z(1, H, D, D, dtype=F32)), ValueError, "state_in"),
    (dict(state_out=z(B, H, D, D - 1, dtype=F32)), ValueError, "state_out"),
])
def test_prefill_argument_mismatch(kw, exc, name):
    args = dict(slopes=z(H, dtype=F32))
    args.update(kw)
    slopes = args.pop("slopes")
    state_in = args.pop("state_in", None)
    raises(lambda: la.lt_prefill(*qkv4(), slopes, 64, state_in, **args), exc, name)
    raises(lambda: la.lt_prefill_noalloc(*qkv4(), slopes, 64, state_in, **args), exc, name)


def test_prefill_qkv_mismatch():
    q, k, v = qkv4()
    raises(lambda: la.lt_prefill(q, k[:, :4], v, z(H, dtype=F32), 64), ValueError, "q, k, v")
    raises(lambda: la.lt_prefill(q, k.float(), v, z(H, dtype=F32), 64), TypeError, "q, k, v")
    raises(lambda: la.lt_prefill(q.to(torch.float16), k.to(torch.float16), v.to(torch.float16),
                                 z(H, dtype=F32), 64), TypeError, "q")


@pytest.mark.parametrize("kw,exc,name", [
    (dict(cu=torch.tensor([0, 3, 8], dtype=torch.int64)), TypeError, "cu_seqlens"),
    (dict(o=z(7, H, D, dtype=F32)), ValueError, "o"),
    (dict(state_in=z(3, H, D, D, dtype=F32)), ValueError, "state_in"),  # 2 sequences
    (dict(slopes=z(H)), TypeError, "slopes"),
    (dict(workspace=z(4, 4, dtype=torch.uint8).t()), ValueError, "workspace"),  # not contiguous
])
def test_varlen_argument_mismatch(kw, exc, name):
    q, k, v = z(8, H, D), z(8, H, D), z(8, H, D)
    cu = kw.pop("cu", torch.tensor([0, 3, 8], dtype=torch.int32))
    slopes = kw.pop("slopes", z(H, dtype=F32))
    state_in = kw.pop("state_in", None)
    raises(lambda: la.lt_prefill_varlen(q, k, v, cu, slopes, 64, state_in, max_seqlen=5, **kw), exc, name)


@pytest.mark.parametrize("kw,exc,name", [
    (dict(state=z(B, H, D, D)), TypeError, "state"),
    (dict(state=z(B + 1, H, D, D, dtype=F32)), ValueError, "state"),
    (dict(o=z(B, H, D - 1, dtype=F32)), ValueError, "o"),
    (dict(slopes=z(H, dtype=torch.float64)), TypeError, "slopes"),
])
def test_decode_argument_mismatch(kw, exc, name):
    q, k, v = z(B, H, D), z(B, H, D), z(B, H, D)
    state = kw.pop("state", z(B, H, D, D, dtype=F32))
    slopes = kw.pop("slopes", z(H, dtype=F32))
    raises(lambda: la.lt_decode(q, k, v, slopes, state, **kw), exc, name)


def test_decode_slots_argument_mismatch():
    q, k, v = z(B, H, D), z(B, H, D), z(B, H, D)
    sl = z(H, dtype=F32)
    pool = z(5, H, D, D, dtype=F32)
    raises(lambda: la.lt_decode_slots(q, k, v, sl, pool, torch.zeros(B, dtype=torch.int64)), TypeError, "slot_ids")
    raises(lambda: la.lt_decode_slots(q, k, v, sl, pool, torch.zeros(B + 1, dtype=torch.int32)), ValueError,
           "slot_ids")
    raises(lambda: la.lt_decode_slots(q, k, v, sl, z(5, H + 1, D, D, dtype=F32), torch.zeros(B, dtype=torch.int32)),
           ValueError, "state_pool")


@pytest.mark.parametrize("which,bad,exc", [
    ("gate", z(B, L, H, D, dtype=F32), TypeError),
    ("gate", z(B, L, H - 1, D), ValueError),
    ("norm_weight", z(H, D), TypeError),
    ("norm_weight", z(H + 1, D, dtype=F32), ValueError),
])
def test_norm_gate_argument_mismatch(which, bad, exc):
    args = dict(gate=z(B, L, H, D), norm_weight=z(H, D, dtype=F32))
    args[which] = bad
    raises(lambda: la.lt_prefill_norm_gate(*qkv4(), z(H, dtype=F32), args["gate"], args["norm_weight"], 1e-6, 64),
           exc, which)
    q1, k1, v1 = z(B, H, D), z(B, H, D), z(B, H, D)
    g1 = args["gate"][:, 0] if args["gate"].dim() == 4 else args["gate"]
    raises(lambda: la.lt_decode_norm_gate(q1, k1, v1, z(H, dtype=F32), z(B, H, D, D, dtype=F32),
                                          g1.contiguous(), args["norm_weight"], 1e-6), exc, which)


@pytest.mark.parametrize("kw,exc,name", [
    (dict(dq=z(B, L, H, D, dtype=F32), dk=z(B, L, H, D)), TypeError, "dk"),  # bf16 dk beside fp32 dq
    (dict(dq=z(B, L, H, D, dtype=F32), dv=z(B, L, H, D)), TypeError, "dv"),
    (dict(dq=z(B, L - 1, H, D, dtype=F32)), ValueError, "dq"),
    (dict(d_state_out=z(B, H, D, 64, dtype=F32)), ValueError, "d_state_out"),
    (dict(d_state_in=z(B, H, D, D)), TypeError, "d_state_in"),
])
def test_backward_argument_mismatch(kw, exc, name):
    q, k, v = qkv4()
    do = z(B, L, H, D)
    d_state_out = kw.pop("d_state_out", None)
    raises(lambda: la.lt_prefill_backward(q, k, v, do, z(H, dtype=F32), 64, None, d_state_out, **kw), exc, name)


def test_backward_grad_dtype_disagreement():
    q, k, v = qkv4()
    raises(lambda: la.lt_prefill_backward(q, k, v, z(B, L, H, D), z(H, dtype=F32), 64,
                                          dq=z(B, L, H, D, dtype=F32), grad_dtype=BF), TypeError, "dq, dk and dv")


def test_softmax_argument_mismatch():
    q, k, v = z(1, L, 8, D), z(1, L, 2, D), z(1, L, 2, D)
    raises(lambda: la.lt_softmax_prefill(q, k, v, o=z(1, L, 8, 64, dtype=F32)), ValueError, "o")
    raises(lambda: la.lt_softmax_prefill(q, k, v, k_rope=z(1, L, 2, D, dtype=F32)), TypeError, "k_rope")
    raises(lambda: la.lt_softmax_prefill(q.float(), k, v), TypeError, "q")
    qd, kn, vn = z(2, 8, D), z(2, 2, D), z(2, 2, D)
    kc, vc = z(2, 16, 2, D), z(2, 16, 2, D)
    raises(lambda: la.lt_softmax_decode(qd, kn, vn, kc, vc, torch.zeros(2, dtype=torch.int64)), TypeError,
           "lengths")
    raises(lambda: la.lt_softmax_decode(qd, kn, vn, kc, vc, torch.zeros(2, dtype=torch.int32),
                                        o=z(2, 8, D + 1, dtype=F32)), ValueError, "o")
    raises(lambda: la.lt_softmax_decode(qd, kn, vn, kc.float(), vc, torch.zeros(2, dtype=torch.int32)),
           TypeError, "k_cache")
    raises(lambda: la.lt_softmax_decode(qd, kn, vn, kc, vc[:, :8], torch.zeros(2, dtype=torch.int32)),
           ValueError, "caches")
