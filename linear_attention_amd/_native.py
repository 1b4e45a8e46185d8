"""ctypes binding of ``liblightning.so`` (the C ABI in ``include/lightning.h``).

Argument marshalling only: shapes and dtypes are read off torch tensors, raw
device pointers and the current HIP stream are passed to the C entry points,
and every step of the computation runs in the library's HIP kernels. There is
no fallback: if the library is missing, importing this module fails.
"""

from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblightning.so")

(LT_OK, LT_ERR_NULL, LT_ERR_SHAPE, LT_ERR_BLOCK, LT_ERR_DTYPE, LT_ERR_ALIAS, LT_ERR_HIP, LT_ERR_VALUE,
 LT_ERR_SCRATCH) = range(9)
LT_F32, LT_BF16 = 0, 1
LT_MAX_BLOCK = 65536
HEAD_DIM = 128

EXPORTS = ("lt_status_string", "lt_version", "lt_build_id", "lt_init", "lt_prefill", "lt_prefill_noalloc",
           "lt_prefill_workspace_bytes", "lt_prefill_varlen", "lt_prefill_varlen_workspace_bytes",
           "lt_decode", "lt_prefill_norm_gate", "lt_prefill_varlen_norm_gate",
           "lt_decode_norm_gate", "lt_decode_slots", "lt_prefill_backward", "lt_softmax_prefill",
           "lt_softmax_decode", "lt_softmax_decode_workspace_bytes")

_vp, _i, _ll, _f, _d = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_float, ctypes.c_double


class LightningError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m linear_attention_amd.build` "
            "(the Lightning kernels have no fallback path)")
    # PyTorch for ROCm ships its own HIP runtime. Loading torch first lets the
    # library's libamdhip64.so.7 dependency resolve to that same runtime; loaded
    # the other way round, the process would hold two HIP runtimes, and the one
    # the library uses reports no device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    lib.lt_status_string.argtypes = [_i]
    lib.lt_status_string.restype = ctypes.c_char_p
    lib.lt_version.argtypes = []
    lib.lt_version.restype = _i
    lib.lt_build_id.argtypes = []
    lib.lt_build_id.restype = ctypes.c_char_p
    lib.lt_init.argtypes = []
    lib.lt_init.restype = _i
    lib.lt_prefill.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _vp,
                               _i, _ll, _i, _i, _i, _vp, ctypes.c_size_t, _vp]
    lib.lt_prefill.restype = _i
    lib.lt_prefill_noalloc.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _vp,
                                       _i, _ll, _i, _i, _i, _vp]
    lib.lt_prefill_noalloc.restype = _i
    lib.lt_prefill_workspace_bytes.argtypes = [_i, _ll, _i, _i, _i]
    lib.lt_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.lt_prefill_varlen.argtypes = [_vp, _vp, _vp, _i, _vp, _i, _ll, _ll, _vp, _vp, _i,
                                      _vp, _vp, _i, _i, _i, _vp, ctypes.c_size_t, _vp]
    lib.lt_prefill_varlen.restype = _i
    lib.lt_prefill_varlen_workspace_bytes.argtypes = [_i, _ll, _i, _i, _i]
    lib.lt_prefill_varlen_workspace_bytes.restype = ctypes.c_size_t
    lib.lt_decode.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _i, _vp]
    lib.lt_decode.restype = _i
    lib.lt_prefill_norm_gate.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _f, _vp, _i, _vp, _vp,
                                         _i, _ll, _i, _i, _i, _vp, ctypes.c_size_t, _vp]
    lib.lt_prefill_norm_gate.restype = _i
    lib.lt_prefill_varlen_norm_gate.argtypes = [_vp, _vp, _vp, _i, _vp, _i, _ll, _ll, _vp, _vp, _vp, _f,
                                                _vp, _i, _vp, _vp, _i, _i, _i, _vp, ctypes.c_size_t,
                                                _vp]
    lib.lt_prefill_varlen_norm_gate.restype = _i
    lib.lt_decode_norm_gate.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _f, _vp, _i, _i, _i,
                                        _i, _vp]
    lib.lt_decode_norm_gate.restype = _i
    lib.lt_decode_slots.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _vp]
    lib.lt_decode_slots.restype = _i
    lib.lt_prefill_backward.argtypes = [_vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp,
                                        _i, _ll, _i, _i, _i, _vp, ctypes.c_size_t, _vp]
    lib.lt_prefill_backward.restype = _i
    lib.lt_softmax_prefill.argtypes = [_vp, _vp, _vp, _vp, _i, _vp, _i, _ll, _i, _i, _i, _i, _d, _f,
                                       _ll, _vp]
    lib.lt_softmax_prefill.restype = _i
    lib.lt_softmax_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _ll, _i, _i, _i, _i, _d,
                                      _f, _vp, ctypes.c_size_t, _vp]
    lib.lt_softmax_decode.restype = _i
    lib.lt_softmax_decode_workspace_bytes.argtypes = [_i, _ll, _i, _i, _i]
    lib.lt_softmax_decode_workspace_bytes.restype = ctypes.c_size_t
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.lt_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != LT_OK:
        raise LightningError(status, where)


def lt_init() -> None:
    """Optional set-up on the current device: loads the library's GPU code
    (otherwise loaded inside the first call of each kernel source) and looks up
    the no-allocation scratch. Raises LightningError without a device."""
    _check(lib.lt_init(), "lt_init")


# ---------------------------------------------------------------------------
# torch-facing wrappers (same names as the C entry points)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t == torch.float32:
        return LT_F32
    if t == torch.bfloat16:
        return LT_BF16
    raise TypeError(f"unsupported dtype {t}; Lightning kernels take float32 or bfloat16")


class _Args:
    """The tensor arguments of one call. ``ptrs()`` checks every shape, dtype and
    layout, then every device, before any raw pointer reaches the library:
    a wrong-sized or wrongly typed buffer would otherwise be read or written
    out of bounds on the device (the C ABI sees only pointers and sizes)."""

    def __init__(self, device):
        self.device = device
        self.items = []

    def add(self, t, name, shape=None, dtypes=None):
        self.items.append((t, name, None if shape is None else tuple(int(x) for x in shape), dtypes))
        return self

    def ptrs(self):
        for t, name, shape, dtypes in self.items:
            if t is None:
                continue
            if shape is not None and tuple(t.shape) != shape:
                raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
            if dtypes is not None and t.dtype not in dtypes:
                names = " or ".join(str(d) for d in dtypes)
                raise TypeError(f"{name} must be {names}, got {t.dtype}")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        for t, name, _, _ in self.items:
            if t is None:
                continue
            if not t.is_cuda:
                raise ValueError(f"{name} must be a device tensor")
            if t.device != self.device:
                raise ValueError(f"{name} is on {t.device}, the call's inputs on {self.device}")
        return [None if t is None else t.data_ptr() for t, _, _, _ in self.items]


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _io_dtypes():
    torch = _torch()
    return (torch.float32, torch.bfloat16)


def _out(t, shape, out_dtype, like, name):
    """The caller's output tensor (whose dtype must agree with out_dtype when both
    are given), or a new one of out_dtype (default float32)."""
    torch = _torch()
    if t is not None:
        if out_dtype is not None and t.dtype != out_dtype:
            raise TypeError(f"{name} is {t.dtype} but out_dtype is {out_dtype}")
        return t
    return torch.empty(shape, device=like.device, dtype=out_dtype or torch.float32)


def _qkv(q, k, v, ndim, what):
    if q.dim() != ndim or k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q, k, v must share one {what} shape")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if q.dtype not in _io_dtypes():
        raise TypeError(f"q, k, v must be float32 or bfloat16, got {q.dtype}")


def lt_prefill_workspace_bytes(batch, seqlen, heads, head_dim=HEAD_DIM, in_dtype=LT_BF16) -> int:
    return int(lib.lt_prefill_workspace_bytes(int(batch), int(seqlen), int(heads), int(head_dim),
                                              int(in_dtype)))


def lt_prefill_varlen_workspace_bytes(num_seqs, max_seqlen, heads, head_dim=HEAD_DIM, in_dtype=LT_BF16) -> int:
    return int(lib.lt_prefill_varlen_workspace_bytes(int(num_seqs), int(max_seqlen), int(heads),
                                                     int(head_dim), int(in_dtype)))


def _prefill_args(q, k, v, slopes, o, state_in, state_out, extra=()):
    """Checked pointers of a fixed-length prefill's tensors (q, k, v, slopes, o,
    state_in, state_out, then `extra` (tensor, name, shape, dtypes) entries)."""
    torch = _torch()
    batch, L, H, d = q.shape
    a = _Args(q.device)
    a.add(q, "q", dtypes=_io_dtypes()).add(k, "k").add(v, "v")
    a.add(slopes, "slopes", (H,), (torch.float32,))
    a.add(o, "o", (batch, L, H, d), _io_dtypes())
    a.add(state_in, "state_in", (batch, H, d, d), (torch.float32,))
    a.add(state_out, "state_out", (batch, H, d, d), (torch.float32,))
    for e in extra:
        a.add(*e)
    return a.ptrs()


def lt_prefill(q, k, v, slopes, block, state_in=None, *, o=None, state_out=None,
               want_state=True, out_dtype=None, workspace=None, stream=None):
    """Fixed-length prefill. q, k, v: [batch, L, H, 128]; slopes: fp32 [H].

    Returns (o [batch, L, H, 128], state_out [batch, H, 128, 128] fp32 or None).
    ``state_out`` may be given (it may be ``state_in`` itself for an in-place
    update); otherwise one is allocated when ``want_state``. ``workspace`` is a
    device tensor of at least ``lt_prefill_workspace_bytes`` bytes; one is
    allocated when it is None and the plan wants one.
    """
    torch = _torch()
    _qkv(q, k, v, 4, "[batch, L, H, d]")
    batch, L, H, d = q.shape
    o = _out(o, (batch, L, H, d), out_dtype, q, "o")
    if state_out is None and want_state:
        state_out = torch.empty((batch, H, d, d), device=q.device, dtype=torch.float32)
    if workspace is None:
        nbytes = lt_prefill_workspace_bytes(batch, L, H, d, _dtype_code(q.dtype))
        if nbytes:
            workspace = torch.empty(nbytes, device=q.device, dtype=torch.uint8)
    p = _prefill_args(q, k, v, slopes, o, state_in, state_out, [(workspace, "workspace")])
    st = lib.lt_prefill(p[0], p[1], p[2], _dtype_code(q.dtype), p[3], p[4], _dtype_code(o.dtype),
                        p[5], p[6], batch, L, H, d, int(block), p[7], _nbytes(workspace),
                        _stream(stream, q.device))
    _check(st, "lt_prefill")
    return o, state_out


def lt_prefill_noalloc(q, k, v, slopes, block, state_in=None, *, o=None, state_out=None,
                       want_state=True, out_dtype=None, stream=None):
    """lt_prefill without a workspace argument: the library's static scratch
    (64 MiB per GPU, held from the first call on a GPU until the process ends)
    serves the split of long sequences. Calls whose work overlaps on one GPU
    race on that scratch. Same arguments and result as lt_prefill otherwise.
    """
    torch = _torch()
    _qkv(q, k, v, 4, "[batch, L, H, d]")
    batch, L, H, d = q.shape
    o = _out(o, (batch, L, H, d), out_dtype, q, "o")
    if state_out is None and want_state:
        state_out = torch.empty((batch, H, d, d), device=q.device, dtype=torch.float32)
    p = _prefill_args(q, k, v, slopes, o, state_in, state_out)
    st = lib.lt_prefill_noalloc(p[0], p[1], p[2], _dtype_code(q.dtype), p[3], p[4], _dtype_code(o.dtype),
                                p[5], p[6], batch, L, H, d, int(block), _stream(stream, q.device))
    _check(st, "lt_prefill_noalloc")
    return o, state_out


def _varlen_args(q, k, v, cu_seqlens, slopes, o, state_in, state_out, extra=()):
    torch = _torch()
    T, H, d = q.shape
    n = cu_seqlens.numel() - 1
    a = _Args(q.device)
    a.add(q, "q", dtypes=_io_dtypes()).add(k, "k").add(v, "v")
    a.add(cu_seqlens, "cu_seqlens", (n + 1,), (torch.int32,))
    a.add(slopes, "slopes", (H,), (torch.float32,))
    a.add(o, "o", (T, H, d), _io_dtypes())
    a.add(state_in, "state_in", (n, H, d, d), (torch.float32,))
    a.add(state_out, "state_out", (n, H, d, d), (torch.float32,))
    for e in extra:
        a.add(*e)
    return a.ptrs()


def _varlen_common(q, k, v, cu_seqlens, max_seqlen, want_state, state_out, workspace):
    torch = _torch()
    _qkv(q, k, v, 3, "[T, H, d]")
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D tensor of num_seqs + 1 entries")
    T, H, d = q.shape
    n = cu_seqlens.numel() - 1
    if max_seqlen is None:
        max_seqlen = T  # an upper bound (the split is then cut on it)
    if state_out is None and want_state:
        state_out = torch.empty((n, H, d, d), device=q.device, dtype=torch.float32)
    if workspace is None:
        nbytes = lt_prefill_varlen_workspace_bytes(n, max_seqlen, H, d, _dtype_code(q.dtype))
        if nbytes:
            workspace = torch.empty(nbytes, device=q.device, dtype=torch.uint8)
    return T, H, d, n, int(max_seqlen), state_out, workspace


def lt_prefill_varlen(q, k, v, cu_seqlens, slopes, block, state_in=None, *, max_seqlen=None, o=None,
                      state_out=None, want_state=True, out_dtype=None, workspace=None, stream=None):
    """Packed variable-length prefill. q, k, v: [T, H, 128]; cu_seqlens: int32 [n+1] on device.

    max_seqlen: the longest sequence's length (None: T, an upper bound). A
    workspace of lt_prefill_varlen_workspace_bytes bytes is allocated when none
    is given and the plan wants one.
    Returns (o [T, H, 128], state_out [n, H, 128, 128] fp32 or None).
    """
    T, H, d, n, mx, state_out, workspace = _varlen_common(q, k, v, cu_seqlens, max_seqlen, want_state,
                                                          state_out, workspace)
    o = _out(o, (T, H, d), out_dtype, q, "o")
    p = _varlen_args(q, k, v, cu_seqlens, slopes, o, state_in, state_out, [(workspace, "workspace")])
    st = lib.lt_prefill_varlen(p[0], p[1], p[2], _dtype_code(q.dtype), p[3], n, T, mx, p[4], p[5],
                               _dtype_code(o.dtype), p[6], p[7], H, d, int(block), p[8],
                               _nbytes(workspace), _stream(stream, q.device))
    _check(st, "lt_prefill_varlen")
    return o, state_out


def _decode_args(q, k, v, slopes, state, o, state_shape, state_name="state", extra=()):
    torch = _torch()
    batch, H, d = q.shape
    a = _Args(q.device)
    a.add(q, "q", dtypes=_io_dtypes()).add(k, "k").add(v, "v")
    a.add(slopes, "slopes", (H,), (torch.float32,))
    a.add(state, state_name, state_shape, (torch.float32,))
    a.add(o, "o", (batch, H, d), _io_dtypes())
    for e in extra:
        a.add(*e)
    return a.ptrs()


def lt_decode(q, k, v, slopes, state, *, o=None, out_dtype=None, stream=None):
    """One decode step. q, k, v: [batch, H, 128]; state: [batch, H, 128, 128] fp32, updated in place.

    Returns o [batch, H, 128].
    """
    _qkv(q, k, v, 3, "[batch, H, d]")
    batch, H, d = q.shape
    o = _out(o, (batch, H, d), out_dtype, q, "o")
    p = _decode_args(q, k, v, slopes, state, o, (batch, H, d, d))
    st = lib.lt_decode(p[0], p[1], p[2], _dtype_code(q.dtype), p[3], p[4], p[5], _dtype_code(o.dtype),
                       batch, H, d, _stream(stream, q.device))
    _check(st, "lt_decode")
    return o


def _gate_entries(gate, norm_weight, like, H):
    torch = _torch()
    return [(gate, "gate", tuple(like.shape), (like.dtype,)),
            (norm_weight, "norm_weight", (H, HEAD_DIM), (torch.float32,))]


def lt_prefill_norm_gate(q, k, v, slopes, gate, norm_weight, eps, block, state_in=None, *, y=None,
                         state_out=None, want_state=True, out_dtype=None, workspace=None,
                         stream=None):
    """Fixed-length prefill followed by y = rmsnorm(o) * norm_weight * sigmoid(gate) per
    (token, head). q, k, v, gate: bf16 [batch, L, H, 128]; norm_weight: fp32 [H, 128].

    Returns (y [batch, L, H, 128], state_out or None); other arguments as lt_prefill.
    """
    torch = _torch()
    _qkv(q, k, v, 4, "[batch, L, H, d]")
    batch, L, H, d = q.shape
    y = _out(y, (batch, L, H, d), out_dtype, q, "y")
    if state_out is None and want_state:
        state_out = torch.empty((batch, H, d, d), device=q.device, dtype=torch.float32)
    if workspace is None:
        nbytes = lt_prefill_workspace_bytes(batch, L, H, d, _dtype_code(q.dtype))
        if nbytes:
            workspace = torch.empty(nbytes, device=q.device, dtype=torch.uint8)
    p = _prefill_args(q, k, v, slopes, y, state_in, state_out,
                      _gate_entries(gate, norm_weight, q, H) + [(workspace, "workspace")])
    st = lib.lt_prefill_norm_gate(p[0], p[1], p[2], _dtype_code(q.dtype), p[3], p[7], p[8], float(eps), p[4],
                                  _dtype_code(y.dtype), p[5], p[6], batch, L, H, d, int(block), p[9],
                                  _nbytes(workspace), _stream(stream, q.device))
    _check(st, "lt_prefill_norm_gate")
    return y, state_out


def lt_prefill_varlen_norm_gate(q, k, v, cu_seqlens, slopes, gate, norm_weight, eps, block,
                                state_in=None, *, max_seqlen=None, y=None, state_out=None,
                                want_state=True, out_dtype=None, workspace=None, stream=None):
    """Packed variable-length prefill followed by the norm-gate epilogue.
    q, k, v, gate: bf16 [T, H, 128]; other arguments as lt_prefill_varlen.

    Returns (y [T, H, 128], state_out [n, H, 128, 128] or None).
    """
    T, H, d, n, mx, state_out, workspace = _varlen_common(q, k, v, cu_seqlens, max_seqlen, want_state,
                                                          state_out, workspace)
    y = _out(y, (T, H, d), out_dtype, q, "y")
    p = _varlen_args(q, k, v, cu_seqlens, slopes, y, state_in, state_out,
                     _gate_entries(gate, norm_weight, q, H) + [(workspace, "workspace")])
    st = lib.lt_prefill_varlen_norm_gate(
        p[0], p[1], p[2], _dtype_code(q.dtype), p[3], n, T, mx, p[4], p[8], p[9], float(eps), p[5],
        _dtype_code(y.dtype), p[6], p[7], H, d, int(block), p[10], _nbytes(workspace),
        _stream(stream, q.device))
    _check(st, "lt_prefill_varlen_norm_gate")
    return y, state_out


def lt_decode_norm_gate(q, k, v, slopes, state, gate, norm_weight, eps, *, y=None, out_dtype=None,
                        stream=None):
    """One decode step followed by the norm-gate epilogue. q, k, v, gate: [batch, H, 128];
    state: [batch, H, 128, 128] fp32, updated in place. Returns y [batch, H, 128].
    """
    _qkv(q, k, v, 3, "[batch, H, d]")
    batch, H, d = q.shape
    y = _out(y, (batch, H, d), out_dtype, q, "y")
    p = _decode_args(q, k, v, slopes, state, y, (batch, H, d, d),
                     extra=_gate_entries(gate, norm_weight, q, H))
    st = lib.lt_decode_norm_gate(p[0], p[1], p[2], _dtype_code(q.dtype), p[3], p[4], p[6], p[7],
                                 float(eps), p[5], _dtype_code(y.dtype), batch, H, d,
                                 _stream(stream, q.device))
    _check(st, "lt_decode_norm_gate")
    return y


def lt_decode_slots(q, k, v, slopes, state_pool, slot_ids, *, o=None, out_dtype=None, stream=None):
    """One decode step over a state pool. q, k, v: [batch, H, 128]; state_pool:
    [num_slots, H, 128, 128] fp32, updated in place; slot_ids: int32 [batch] on the
    device (out-of-range ids are padding rows with zero output). Returns o [batch, H, 128].
    """
    torch = _torch()
    _qkv(q, k, v, 3, "[batch, H, d]")
    batch, H, d = q.shape
    if state_pool.dim() != 4:
        raise ValueError("state_pool must be [num_slots, H, d, d]")
    slots = int(state_pool.shape[0])
    o = _out(o, (batch, H, d), out_dtype, q, "o")
    p = _decode_args(q, k, v, slopes, state_pool, o, (slots, H, d, d), "state_pool",
                     [(slot_ids, "slot_ids", (batch,), (torch.int32,))])
    st = lib.lt_decode_slots(p[0], p[1], p[2], _dtype_code(q.dtype), p[3], p[4], slots, p[6], p[5],
                             _dtype_code(o.dtype), batch, H, d, _stream(stream, q.device))
    _check(st, "lt_decode_slots")
    return o


def lt_prefill_backward(q, k, v, dout, slopes, block, state_in=None, d_state_out=None, *, dq=None,
                        dk=None, dv=None, d_state_in=None, want_d_state_in=True, grad_dtype=None,
                        workspace=None, stream=None):
    """Gradients of sum(dout * o) + <d_state_out, S_final> for a fixed-length prefill.
    q, k, v, dout: bf16 [batch, L, H, 128]; state_in, d_state_out: fp32 [batch, H, 128, 128]
    or None. Returns (dq, dk, dv [batch, L, H, 128] in grad_dtype (default fp32, or the
    dtype of the given gradient tensors, which must agree), d_state_in [batch, H, 128, 128]
    fp32 or None).
    """
    torch = _torch()
    if q.dim() != 4 or any(x.shape != q.shape for x in (k, v, dout)):
        raise ValueError("q, k, v, dout must share one [batch, L, H, d] shape")
    if any(x.dtype != q.dtype for x in (k, v, dout)):
        raise TypeError("q, k, v, dout must share one dtype")
    batch, L, H, d = q.shape
    given = [g.dtype for g in (dq, dk, dv) if g is not None]
    if grad_dtype is None:
        grad_dtype = given[0] if given else torch.float32
    if any(g != grad_dtype for g in given):
        raise TypeError(f"dq, dk and dv must all be {grad_dtype}")
    mk = lambda: torch.empty((batch, L, H, d), device=q.device, dtype=grad_dtype)
    dq = mk() if dq is None else dq
    dk = mk() if dk is None else dk
    dv = mk() if dv is None else dv
    if d_state_in is None and want_d_state_in:
        d_state_in = torch.empty((batch, H, d, d), device=q.device, dtype=torch.float32)
    if workspace is None:
        nbytes = lt_prefill_workspace_bytes(batch, L, H, d, _dtype_code(q.dtype))
        if nbytes:
            workspace = torch.empty(nbytes, device=q.device, dtype=torch.uint8)
    sh, st_sh = (batch, L, H, d), (batch, H, d, d)
    a = _Args(q.device)
    a.add(q, "q", dtypes=(torch.bfloat16,)).add(k, "k").add(v, "v").add(dout, "dout")
    a.add(slopes, "slopes", (H,), (torch.float32,))
    a.add(state_in, "state_in", st_sh, (torch.float32,))
    a.add(d_state_out, "d_state_out", st_sh, (torch.float32,))
    a.add(dq, "dq", sh, (grad_dtype,)).add(dk, "dk", sh, (grad_dtype,)).add(dv, "dv", sh, (grad_dtype,))
    a.add(d_state_in, "d_state_in", st_sh, (torch.float32,))
    a.add(workspace, "workspace")
    p = a.ptrs()
    st = lib.lt_prefill_backward(p[0], p[1], p[2], p[3], _dtype_code(q.dtype), p[4], p[5], p[6], p[7],
                                 p[8], p[9], _dtype_code(grad_dtype), p[10], batch, L, H, d, int(block),
                                 p[11], _nbytes(workspace), _stream(stream, q.device))
    _check(st, "lt_prefill_backward")
    return dq, dk, dv, d_state_in


def lt_softmax_prefill(q, k, v, *, rope_dims=64, rope_base=10000.0, scale=None, pos0=0, o=None,
                       out_dtype=None, k_rope=None, stream=None):
    """Causal softmax attention with grouped K/V heads and partial RoPE.
    q: bf16 [batch, L, Hq, 128]; k, v: bf16 [batch, L, Hkv, 128]. Returns
    (o [batch, L, Hq, 128] in out_dtype (default fp32), k_rope = rope(k) bf16).
    """
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]:
        raise ValueError("q must be [batch, L, Hq, d] and k, v [batch, L, Hkv, d]")
    batch, L, Hq, d = q.shape
    Hkv = k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = _out(o, (batch, L, Hq, d), out_dtype, q, "o")
    if k_rope is None:
        k_rope = torch.empty_like(k)
    bf = (torch.bfloat16,)
    p = (_Args(q.device).add(q, "q", dtypes=bf).add(k, "k", dtypes=bf).add(v, "v", dtypes=bf)
         .add(o, "o", (batch, L, Hq, d), _io_dtypes()).add(k_rope, "k_rope", tuple(k.shape), bf).ptrs())
    st = lib.lt_softmax_prefill(p[0], p[1], p[2], p[3], _dtype_code(o.dtype), p[4], batch, L, Hq, Hkv, d,
                                int(rope_dims), float(rope_base), scale, int(pos0), _stream(stream, q.device))
    _check(st, "lt_softmax_prefill")
    return o, k_rope


def lt_softmax_decode_workspace_bytes(batch, capacity, q_heads, kv_heads, head_dim=128):
    return int(lib.lt_softmax_decode_workspace_bytes(batch, capacity, q_heads, kv_heads, head_dim))


def lt_softmax_decode(q, k_new, v_new, k_cache, v_cache, lengths, *, rope_dims=64, rope_base=10000.0,
                      scale=None, o=None, out_dtype=None, workspace=None, stream=None):
    """One decode step of the softmax layer. q: bf16 [batch, Hq, 128]; k_new, v_new:
    bf16 [batch, Hkv, 128]; k_cache, v_cache: bf16 [batch, capacity, Hkv, 128],
    updated in place at row lengths[b]; lengths: int32 [batch] on the device.
    Returns o [batch, Hq, 128] in out_dtype (default fp32). A workspace is
    allocated here when none is given.
    """
    torch = _torch()
    if q.dim() != 3 or k_new.dim() != 3 or v_new.shape != k_new.shape or k_new.shape[0] != q.shape[0]:
        raise ValueError("q must be [batch, Hq, d] and k_new, v_new [batch, Hkv, d]")
    batch, Hq, d = q.shape
    Hkv = k_new.shape[1]
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape or k_cache.shape[0] != batch or \
            tuple(k_cache.shape[2:]) != (Hkv, d):
        raise ValueError("caches must be [batch, capacity, Hkv, d]")
    cap = k_cache.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = _out(o, (batch, Hq, d), out_dtype, q, "o")
    if workspace is None:
        nb = lt_softmax_decode_workspace_bytes(batch, cap, Hq, Hkv, d)
        workspace = torch.empty(max(nb, 1), device=q.device, dtype=torch.uint8) if nb else None
    bf = (torch.bfloat16,)
    p = (_Args(q.device).add(q, "q", dtypes=bf).add(k_new, "k_new", dtypes=bf).add(v_new, "v_new", dtypes=bf)
         .add(k_cache, "k_cache", dtypes=bf).add(v_cache, "v_cache", dtypes=bf)
         .add(lengths, "lengths", (batch,), (torch.int32,)).add(o, "o", (batch, Hq, d), _io_dtypes())
         .add(workspace, "workspace").ptrs())
    st = lib.lt_softmax_decode(p[0], p[1], p[2], p[3], p[4], p[5], p[6], _dtype_code(o.dtype), batch,
                               cap, Hq, Hkv, d, int(rope_dims), float(rope_base), scale, p[7],
                               _nbytes(workspace), _stream(stream, q.device))
    _check(st, "lt_softmax_decode")
    return o
