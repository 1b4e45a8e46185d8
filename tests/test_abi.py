"""The C-ABI library on the CPU: it loads, exports every declared symbol, and its
host-side argument checks return the documented status codes before any HIP
call (no compute is launched here)."""

import os
import re

import pytest

from parity_util import ensure_built

ensure_built()

import linear_attention_amd as la  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lightning.h")

# Fake, never-dereferenced device addresses: every call below fails validation
# (or is a documented no-op) before the library touches HIP.
A = 0x10_0000_0000
MB = 1 << 20


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"LT_API\s+[\w\s\*]+?\b(lt_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_symbols() == sorted(la.EXPORTS)


def test_library_exports_every_declared_symbol():
    for name in declared_symbols():
        assert hasattr(la.lib, name), name


def test_only_the_abi_is_exported():
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", la.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert {s for s in syms if s.startswith("lt_")} == set(la.EXPORTS)


def test_status_strings():
    names = ["LT_OK", "LT_ERR_NULL", "LT_ERR_SHAPE", "LT_ERR_BLOCK", "LT_ERR_DTYPE",
             "LT_ERR_ALIAS", "LT_ERR_HIP", "LT_ERR_VALUE", "LT_ERR_SCRATCH"]
    for code, name in enumerate(names):
        assert la.status_string(code).startswith(name)
        assert getattr(la, name) == code
    assert la.status_string(99) == "unknown lt_status"
    assert la.lib.lt_version() == 20100


def test_init_without_a_device():
    """lt_init reports LT_ERR_HIP, without crashing, where no GPU is visible
    (its loads and the scratch lookup are HIP calls; tests/test_parity_gpu.py
    covers it on a GPU)."""
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: covered by the GPU tests")
    assert la.lib.lt_init() == la.LT_ERR_HIP
    with pytest.raises(la.LightningError):
        la.lt_init()


def test_build_id_matches_the_sources():
    """The library reports the hash of the csrc/ and include/ files it was built
    from (the test fixture rebuilds it when they differ)."""
    from linear_attention_amd import build as b

    assert la.lib.lt_build_id().decode() == b.source_hash()
    assert b.library_is_current()


def prefill(**kw):
    args = dict(q=A, k=A + 100 * MB, v=A + 200 * MB, in_dtype=la.LT_BF16, slopes=A + 300 * MB,
                o=A + 400 * MB, out_dtype=la.LT_F32, state_in=None, state_out=A + 900 * MB,
                batch=1, seqlen=64, heads=2, head_dim=128, block=64, workspace=None,
                workspace_bytes=0, stream=None)
    args.update(kw)
    return la.lib.lt_prefill(*args.values())


def prefill_noalloc(**kw):
    args = dict(q=A, k=A + 100 * MB, v=A + 200 * MB, in_dtype=la.LT_BF16, slopes=A + 300 * MB,
                o=A + 400 * MB, out_dtype=la.LT_F32, state_in=None, state_out=A + 900 * MB,
                batch=1, seqlen=64, heads=2, head_dim=128, block=64, stream=None)
    args.update(kw)
    return la.lib.lt_prefill_noalloc(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), la.LT_ERR_NULL),
    (dict(slopes=None), la.LT_ERR_NULL),
    (dict(head_dim=64), la.LT_ERR_SHAPE),
    (dict(batch=-1), la.LT_ERR_SHAPE),
    (dict(seqlen=1 << 50, heads=64), la.LT_ERR_SHAPE),
    (dict(block=0), la.LT_ERR_BLOCK),
    (dict(in_dtype=7), la.LT_ERR_DTYPE),
    (dict(o=A + 16384), la.LT_ERR_ALIAS),
    (dict(state_out=A + 400 * MB), la.LT_ERR_ALIAS),
    (dict(batch=0), la.LT_OK),                     # documented no-ops, before any HIP call
    (dict(seqlen=0, state_out=None), la.LT_OK),
])
def test_prefill_noalloc_checks_arguments_before_any_hip_call(kw, code):
    """The no-allocation entry point runs lt_prefill's host checks before it
    looks up its scratch (its first HIP call)."""
    assert prefill_noalloc(**kw) == code


def varlen(**kw):
    args = dict(q=A, k=A + 100 * MB, v=A + 200 * MB, in_dtype=la.LT_BF16,
                cu=A + 290 * MB, num_seqs=2, total=64, max_seqlen=40, slopes=A + 300 * MB,
                o=A + 400 * MB, out_dtype=la.LT_F32, state_in=None, state_out=A + 900 * MB, heads=2,
                head_dim=128, block=64, workspace=None, workspace_bytes=0, stream=None)
    args.update(kw)
    return la.lib.lt_prefill_varlen(*args.values())


def decode(**kw):
    args = dict(q=A, k=A + MB, v=A + 2 * MB, in_dtype=la.LT_BF16, slopes=A + 3 * MB,
                state=A + 4 * MB, o=A + 100 * MB, out_dtype=la.LT_F32, batch=2, heads=2,
                head_dim=128, stream=None)
    args.update(kw)
    return la.lib.lt_decode(*args.values())


@pytest.mark.parametrize("field", ["q", "k", "v", "slopes", "o"])
def test_prefill_null_pointers(field):
    assert prefill(**{field: None}) == la.LT_ERR_NULL


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), la.LT_ERR_SHAPE),
    (dict(head_dim=256), la.LT_ERR_SHAPE),
    (dict(heads=-1), la.LT_ERR_SHAPE),
    (dict(batch=-1), la.LT_ERR_SHAPE),
    (dict(seqlen=-5), la.LT_ERR_SHAPE),
    (dict(seqlen=1 << 50, heads=64), la.LT_ERR_SHAPE),  # byte count overflows int64
    (dict(block=0), la.LT_ERR_BLOCK),
    (dict(block=la.LT_MAX_BLOCK + 1), la.LT_ERR_BLOCK),
    (dict(in_dtype=7), la.LT_ERR_DTYPE),
    (dict(out_dtype=-1), la.LT_ERR_DTYPE),
])
def test_prefill_bad_arguments(kw, code):
    assert prefill(**kw) == code


def test_prefill_alias_checks():
    assert prefill(o=A + 16384) == la.LT_ERR_ALIAS               # o inside q (32 KiB)
    assert prefill(state_out=A + 400 * MB) == la.LT_ERR_ALIAS    # state_out on o
    assert prefill(state_out=A + 10) == la.LT_ERR_ALIAS          # state_out inside q
    s = A + 900 * MB
    assert prefill(state_in=s, state_out=s + 4096) == la.LT_ERR_ALIAS  # partial overlap
    assert prefill(state_in=s, state_out=s + 8 * MB, batch=0) == la.LT_OK


def test_prefill_workspace_alias():
    assert prefill(workspace=A + 100, workspace_bytes=4096) == la.LT_ERR_ALIAS   # inside q
    assert prefill(workspace=A + 900 * MB - 16, workspace_bytes=64) == la.LT_ERR_ALIAS  # state_out


def test_workspace_query():
    ws = la.lt_prefill_workspace_bytes
    st = 128 * 128 * 4  # one fp32 state
    # Segmented plan: per (sequence, head) one state per pre-pass piece, one
    # partial state per segment boundary and one for an in-place final state; the
    # query covers the finer of the two pre-pass granularities (2048 pre-pass
    # workgroups for plain prefill, 512 for the norm-gate variants).
    # batch 1, 64 heads, 32K tokens: 4 segments of 8192; 24576 covered tokens
    # in 32 pieces of 768
    assert ws(1, 32768, 64) == 64 * (32 + 4) * st
    # batch 1, 8 heads, 32K tokens: 16 segments of 2048; 30720 covered tokens
    # in 60 pieces of 512 (the shortest piece) at either granularity
    assert ws(1, 32768, 8) == 8 * (60 + 16) * st
    # batch 1, 2 heads, 1M tokens: 128 segments of 8192; 127 * 8192 covered
    # tokens in 1016 pieces of 1024
    assert ws(1, 1 << 20, 2) == 2 * (1016 + 128) * st
    assert ws(1, 3000, 64) == 0           # short: value slices, no workspace
    assert ws(4, 32768, 64) == 0          # 256 (sequence, head) pairs already fill the GPU
    assert ws(1, 2048, 64) == 0           # too short to split
    assert ws(1, 32768, 64, in_dtype=la.LT_F32) == 0
    assert ws(1, 32768, 64, head_dim=64) == 0
    assert ws(0, 32768, 64) == 0


def test_prefill_noops_need_no_gpu():
    assert prefill(batch=0) == la.LT_OK
    assert prefill(heads=0) == la.LT_OK
    # zero tokens with no state to write: nothing to launch; q/k/v/o may be NULL
    assert prefill(seqlen=0, state_out=None, q=None, k=None, v=None, o=None) == la.LT_OK


def test_varlen_checks():
    assert varlen(cu=None) == la.LT_ERR_NULL
    assert varlen(num_seqs=-1) == la.LT_ERR_SHAPE
    assert varlen(total=-1) == la.LT_ERR_SHAPE
    assert varlen(total=1 << 31, heads=1) == la.LT_ERR_SHAPE     # int32 boundaries
    assert varlen(head_dim=96) == la.LT_ERR_SHAPE
    assert varlen(block=0) == la.LT_ERR_BLOCK
    assert varlen(cu=A + 400 * MB) == la.LT_ERR_ALIAS            # cu_seqlens inside o
    assert varlen(num_seqs=0) == la.LT_OK
    assert varlen(total=0, max_seqlen=0, state_out=None, q=None, k=None, v=None, o=None) == la.LT_OK
    assert varlen(max_seqlen=-1) == la.LT_ERR_SHAPE
    assert varlen(max_seqlen=65) == la.LT_ERR_SHAPE               # longer than all tokens
    assert varlen(workspace=A + 100, workspace_bytes=4096) == la.LT_ERR_ALIAS   # inside q
    assert varlen(workspace=A + 290 * MB, workspace_bytes=4096) == la.LT_ERR_ALIAS  # on cu_seqlens


def test_varlen_workspace_query():
    ws = la.lt_prefill_varlen_workspace_bytes
    st = 128 * 128 * 4
    # 2 sequences x 64 heads, longest 131072 tokens: 2 segments of 65536, the
    # first covered by 16 pre-pass pieces of 4096 (2048 pre-pass workgroups)
    assert ws(2, 131072, 64) == 2 * 64 * (16 + 2) * st
    # the fixed-length plan of the same longest length
    assert ws(2, 131072, 64) == la.lt_prefill_workspace_bytes(2, 131072, 64)
    assert ws(16, 65536, 64) == 0          # 1024 (sequence, head) pairs: no split
    assert ws(2, 3000, 64) == 0            # too short to split
    assert ws(0, 100, 64) == 0 and ws(2, 0, 64) == 0 and ws(2, 100, 64, 96) == 0


@pytest.mark.parametrize("field", ["q", "k", "v", "slopes", "state", "o"])
def test_decode_null_pointers(field):
    assert decode(**{field: None}) == la.LT_ERR_NULL


def test_decode_checks():
    assert decode(head_dim=64) == la.LT_ERR_SHAPE
    assert decode(batch=-1) == la.LT_ERR_SHAPE
    assert decode(in_dtype=3) == la.LT_ERR_DTYPE
    assert decode(o=A + 4 * MB + 1000) == la.LT_ERR_ALIAS        # o inside the state
    assert decode(state=A + 512) == la.LT_ERR_ALIAS              # state over q
    assert decode(batch=0) == la.LT_OK
    assert decode(heads=0) == la.LT_OK


# --------------------------------------------------------------------------
# norm-gate variants: the base checks plus eps, gate / weight pointers, overlap
# --------------------------------------------------------------------------

def prefill_ng(**kw):
    args = dict(q=A, k=A + 100 * MB, v=A + 200 * MB, in_dtype=la.LT_BF16, slopes=A + 300 * MB,
                gate=A + 310 * MB, weight=A + 350 * MB, eps=1e-6, y=A + 400 * MB,
                out_dtype=la.LT_F32, state_in=None, state_out=A + 900 * MB, batch=1, seqlen=64,
                heads=2, head_dim=128, block=64, workspace=None, workspace_bytes=0, stream=None)
    args.update(kw)
    return la.lib.lt_prefill_norm_gate(*args.values())


def varlen_ng(**kw):
    args = dict(q=A, k=A + 100 * MB, v=A + 200 * MB, in_dtype=la.LT_BF16, cu=A + 290 * MB,
                num_seqs=2, total=64, max_seqlen=64, slopes=A + 300 * MB, gate=A + 310 * MB,
                weight=A + 350 * MB, eps=1e-6, y=A + 400 * MB, out_dtype=la.LT_F32, state_in=None,
                state_out=A + 900 * MB, heads=2, head_dim=128, block=64, workspace=None,
                workspace_bytes=0, stream=None)
    args.update(kw)
    return la.lib.lt_prefill_varlen_norm_gate(*args.values())


def decode_ng(**kw):
    args = dict(q=A, k=A + MB, v=A + 2 * MB, in_dtype=la.LT_BF16, slopes=A + 3 * MB,
                state=A + 4 * MB, gate=A + 20 * MB, weight=A + 30 * MB, eps=1e-6,
                y=A + 100 * MB, out_dtype=la.LT_F32, batch=2, heads=2, head_dim=128, stream=None)
    args.update(kw)
    return la.lib.lt_decode_norm_gate(*args.values())


@pytest.mark.parametrize("call", [prefill_ng, varlen_ng, decode_ng])
@pytest.mark.parametrize("eps", [-1e-6, float("nan"), float("inf")])
def test_norm_gate_bad_eps(call, eps):
    assert call(eps=eps) == la.LT_ERR_VALUE


@pytest.mark.parametrize("call", [prefill_ng, varlen_ng, decode_ng])
@pytest.mark.parametrize("field", ["gate", "weight"])
def test_norm_gate_null_pointers(call, field):
    assert call(**{field: None}) == la.LT_ERR_NULL


@pytest.mark.parametrize("call", [prefill_ng, varlen_ng])
def test_norm_gate_prefill_takes_bf16_only(call):
    assert call(in_dtype=la.LT_F32) == la.LT_ERR_DTYPE
    assert call(in_dtype=9) == la.LT_ERR_DTYPE


def test_norm_gate_alias_checks():
    assert prefill_ng(y=A + 310 * MB + 64) == la.LT_ERR_ALIAS          # y inside gate (32 KiB)
    assert prefill_ng(weight=A + 400 * MB) == la.LT_ERR_ALIAS          # weight on y
    assert prefill_ng(state_out=A + 350 * MB) == la.LT_ERR_ALIAS       # state_out on weight
    assert prefill_ng(workspace=A + 310 * MB, workspace_bytes=64) == la.LT_ERR_ALIAS  # on gate
    assert varlen_ng(y=A + 310 * MB) == la.LT_ERR_ALIAS
    assert decode_ng(y=A + 20 * MB) == la.LT_ERR_ALIAS                 # y on gate
    assert decode_ng(state=A + 30 * MB) == la.LT_ERR_ALIAS             # state on weight


def test_norm_gate_base_checks_still_apply():
    assert prefill_ng(q=None) == la.LT_ERR_NULL
    assert prefill_ng(block=0) == la.LT_ERR_BLOCK
    assert prefill_ng(head_dim=64) == la.LT_ERR_SHAPE
    assert varlen_ng(cu=None) == la.LT_ERR_NULL
    assert decode_ng(state=None) == la.LT_ERR_NULL
    assert decode_ng(out_dtype=5) == la.LT_ERR_DTYPE


def test_norm_gate_noops_need_no_gpu():
    assert prefill_ng(batch=0) == la.LT_OK
    assert prefill_ng(heads=0) == la.LT_OK
    assert prefill_ng(seqlen=0, state_out=None, gate=None, weight=None) == la.LT_OK
    assert varlen_ng(num_seqs=0, total=0, max_seqlen=0) == la.LT_OK
    assert decode_ng(batch=0, gate=None, weight=None) == la.LT_OK


# --------------------------------------------------------------------------
# decode over a state pool
# --------------------------------------------------------------------------

def decode_slots(**kw):
    args = dict(q=A, k=A + MB, v=A + 2 * MB, in_dtype=la.LT_BF16, slopes=A + 3 * MB,
                pool=A + 10 * MB, num_slots=8, ids=A + 5 * MB, o=A + 200 * MB,
                out_dtype=la.LT_F32, batch=4, heads=2, head_dim=128, stream=None)
    args.update(kw)
    return la.lib.lt_decode_slots(*args.values())


def test_decode_slots_checks():
    assert decode_slots(num_slots=-1) == la.LT_ERR_SHAPE
    assert decode_slots(ids=None) == la.LT_ERR_NULL
    assert decode_slots(pool=None) == la.LT_ERR_NULL
    assert decode_slots(head_dim=64) == la.LT_ERR_SHAPE
    assert decode_slots(in_dtype=3) == la.LT_ERR_DTYPE
    assert decode_slots(o=A + 5 * MB) == la.LT_ERR_ALIAS            # o on slot_ids
    assert decode_slots(ids=A + 10 * MB + 64) == la.LT_ERR_ALIAS     # ids inside the pool
    assert decode_slots(o=A + 10 * MB + 4096) == la.LT_ERR_ALIAS     # o inside the pool (1 MiB)
    assert decode_slots(batch=0) == la.LT_OK
    assert decode_slots(heads=0) == la.LT_OK


def test_one_hip_runtime_per_process():
    """Touching the package before torch (as test collection does) must not
    leave two HIP runtimes in the process (torch ships its own)."""
    import subprocess
    import sys

    code = ("import sys; sys.path.insert(0, %r)\n"
            "import linear_attention_amd as la\n"
            "la.LT_OK; la.lib\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read()\n"
            "print(len({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}))\n") % ROOT
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True)
    assert out.stdout.strip().splitlines()[-1] == "1", out.stdout + out.stderr


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------

def backward(**kw):
    args = dict(q=A, k=A + 100 * MB, v=A + 200 * MB, dout=A + 300 * MB, in_dtype=la.LT_BF16,
                slopes=A + 399 * MB, state_in=None, d_state_out=None, dq=A + 400 * MB,
                dk=A + 500 * MB, dv=A + 600 * MB, grad_dtype=la.LT_F32, d_state_in=A + 900 * MB,
                batch=1, seqlen=64, heads=2, head_dim=128, block=64, workspace=None,
                workspace_bytes=0, stream=None)
    args.update(kw)
    return la.lib.lt_prefill_backward(*args.values())


@pytest.mark.parametrize("field", ["q", "k", "v", "dout", "slopes", "dq", "dk", "dv"])
def test_backward_null_pointers(field):
    assert backward(**{field: None}) == la.LT_ERR_NULL


def test_backward_checks():
    assert backward(in_dtype=la.LT_F32) == la.LT_ERR_DTYPE
    assert backward(grad_dtype=4) == la.LT_ERR_DTYPE
    assert backward(head_dim=64) == la.LT_ERR_SHAPE
    assert backward(seqlen=-1) == la.LT_ERR_SHAPE
    assert backward(block=0) == la.LT_ERR_BLOCK
    assert backward(dq=A + 16) == la.LT_ERR_ALIAS                       # dq inside q
    assert backward(dk=A + 400 * MB + 64) == la.LT_ERR_ALIAS            # dk inside dq (64 KiB)
    assert backward(dv=A + 300 * MB) == la.LT_ERR_ALIAS                 # dv on dout
    assert backward(state_in=A + 900 * MB) == la.LT_ERR_ALIAS           # d_state_in on state_in
    assert backward(d_state_out=A + 900 * MB + 8) == la.LT_ERR_ALIAS
    assert backward(workspace=A + 500 * MB, workspace_bytes=64) == la.LT_ERR_ALIAS
    assert backward(batch=0) == la.LT_OK
    assert backward(heads=0) == la.LT_OK
    assert backward(seqlen=0, d_state_in=None) == la.LT_OK


# --------------------------------------------------------------------------
# softmax attention (grouped K/V heads, partial RoPE)
# --------------------------------------------------------------------------

def softmax_prefill(**kw):
    args = dict(q=A, k=A + 100 * MB, v=A + 200 * MB, o=A + 300 * MB, out_dtype=la.LT_F32,
                k_rope=A + 500 * MB, batch=1, seqlen=64, q_heads=8, kv_heads=2, head_dim=128,
                rope_dims=64, rope_base=10000.0, scale=0.088, pos0=0, stream=None)
    args.update(kw)
    return la.lib.lt_softmax_prefill(*args.values())


@pytest.mark.parametrize("field", ["q", "k", "v", "o", "k_rope"])
def test_softmax_prefill_null_pointers(field):
    assert softmax_prefill(**{field: None}) == la.LT_ERR_NULL


@pytest.mark.parametrize("kw,code", [
    (dict(out_dtype=3), la.LT_ERR_DTYPE),
    (dict(head_dim=64), la.LT_ERR_SHAPE),
    (dict(q_heads=6, kv_heads=4), la.LT_ERR_SHAPE),      # not a multiple
    (dict(q_heads=8, kv_heads=0), la.LT_ERR_SHAPE),
    (dict(rope_dims=48), la.LT_ERR_SHAPE),               # not a multiple of 32
    (dict(rope_dims=160), la.LT_ERR_SHAPE),
    (dict(rope_dims=-32), la.LT_ERR_SHAPE),
    (dict(seqlen=-1), la.LT_ERR_SHAPE),
    (dict(batch=-1), la.LT_ERR_SHAPE),
    (dict(pos0=-5), la.LT_ERR_SHAPE),
    (dict(pos0=(1 << 63) - 10), la.LT_ERR_SHAPE),        # last position overflows
    (dict(seqlen=1 << 40, q_heads=64, kv_heads=8), la.LT_ERR_SHAPE),
    (dict(rope_base=1.0), la.LT_ERR_VALUE),
    (dict(rope_base=float("nan")), la.LT_ERR_VALUE),
    (dict(rope_base=float("inf")), la.LT_ERR_VALUE),
    (dict(scale=0.0), la.LT_ERR_VALUE),
    (dict(scale=float("nan")), la.LT_ERR_VALUE),
    (dict(scale=float("inf")), la.LT_ERR_VALUE),
])
def test_softmax_prefill_bad_arguments(kw, code):
    assert softmax_prefill(**kw) == code


def test_softmax_prefill_alias_checks():
    assert softmax_prefill(o=A + 16) == la.LT_ERR_ALIAS                # o inside q (8 heads, 64 tokens)
    assert softmax_prefill(k_rope=A + 100 * MB + 32) == la.LT_ERR_ALIAS  # k_rope on k
    assert softmax_prefill(k_rope=A + 300 * MB + 64) == la.LT_ERR_ALIAS  # k_rope inside o
    assert softmax_prefill(o=A + 200 * MB + 8) == la.LT_ERR_ALIAS      # o on v


def test_softmax_prefill_noops_need_no_gpu():
    assert softmax_prefill(seqlen=0, q=None) == la.LT_OK
    assert softmax_prefill(batch=0, k=None) == la.LT_OK
    assert softmax_prefill(q_heads=0, kv_heads=0, o=None) == la.LT_OK


def softmax_decode(**kw):
    args = dict(q=A, k_new=A + 10 * MB, v_new=A + 20 * MB, k_cache=A + 100 * MB,
                v_cache=A + 300 * MB, lengths=A + 30 * MB, o=A + 40 * MB, out_dtype=la.LT_F32,
                batch=2, capacity=1000, q_heads=8, kv_heads=2, head_dim=128, rope_dims=64,
                rope_base=10000.0, scale=0.088, workspace=None, workspace_bytes=0, stream=None)
    args.update(kw)
    return la.lib.lt_softmax_decode(*args.values())


@pytest.mark.parametrize("field", ["q", "k_new", "v_new", "k_cache", "v_cache", "lengths", "o"])
def test_softmax_decode_null_pointers(field):
    assert softmax_decode(**{field: None}) == la.LT_ERR_NULL


@pytest.mark.parametrize("kw,code", [
    (dict(out_dtype=2), la.LT_ERR_DTYPE),
    (dict(head_dim=256), la.LT_ERR_SHAPE),
    (dict(q_heads=66, kv_heads=2), la.LT_ERR_SHAPE),     # 33 query heads per K/V head
    (dict(q_heads=9, kv_heads=2), la.LT_ERR_SHAPE),
    (dict(capacity=-1), la.LT_ERR_SHAPE),
    (dict(capacity=1 << 31), la.LT_ERR_SHAPE),           # positions are int32
    (dict(capacity=0), la.LT_ERR_SHAPE),                 # no row for the new token
    (dict(batch=-2), la.LT_ERR_SHAPE),
    (dict(rope_dims=40), la.LT_ERR_SHAPE),
    (dict(rope_base=0.5), la.LT_ERR_VALUE),
    (dict(scale=-1.0), la.LT_ERR_VALUE),
])
def test_softmax_decode_bad_arguments(kw, code):
    assert softmax_decode(**kw) == code


def test_softmax_decode_alias_checks():
    assert softmax_decode(o=A + 8) == la.LT_ERR_ALIAS                    # o on q
    assert softmax_decode(k_cache=A + 10 * MB) == la.LT_ERR_ALIAS        # k_cache on k_new
    assert softmax_decode(v_cache=A + 100 * MB + 4096) == la.LT_ERR_ALIAS  # v_cache inside k_cache
    assert softmax_decode(o=A + 30 * MB) == la.LT_ERR_ALIAS              # o on lengths
    n = la.lt_softmax_decode_workspace_bytes(64, 100000, 8, 2)
    assert n > 0
    big = dict(batch=64, capacity=100000, k_cache=A + 1000 * MB, v_cache=A + 5000 * MB)
    assert softmax_decode(**big, workspace=A + 40 * MB, workspace_bytes=n) == la.LT_ERR_ALIAS  # on o
    assert softmax_decode(**big, workspace=A + 5000 * MB + 64,
                          workspace_bytes=n) == la.LT_ERR_ALIAS            # inside v_cache


def test_softmax_decode_noops_and_workspace_query():
    assert softmax_decode(batch=0, q=None) == la.LT_OK
    assert softmax_decode(q_heads=0, kv_heads=0, o=None) == la.LT_OK
    assert la.lt_softmax_decode_workspace_bytes(16, 33792, 64, 8) == 16 * 64 * 16 * 132 * 4
    assert la.lt_softmax_decode_workspace_bytes(1, 200, 8, 1) == 0       # one split: none needed
    assert la.lt_softmax_decode_workspace_bytes(0, 200, 8, 1) == 0
    assert la.lt_softmax_decode_workspace_bytes(1, 200, 8, 3) == 0       # invalid sizes
