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

EXPORTS = ("lt_status_string", "lt_version", "lt_build_id", "lt_prefill", "lt_prefill_noalloc",
           "lt_prefill_workspace_bytes",
           "lt_prefill_varlen", "lt_decode", "lt_prefill_norm_gate", "lt_prefill_varlen_norm_gate",
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
    lib.lt_prefill.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _vp,
                               _i, _ll, _i, _i, _i, _vp, ctypes.c_size_t, _vp]
    lib.lt_prefill.restype = _i
    lib.lt_prefill_noalloc.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _vp,
                                       _i, _ll, _i, _i, _i, _vp]
    lib.lt_prefill_noalloc.restype = _i
    lib.lt_prefill_workspace_bytes.argtypes = [_i, _ll, _i, _i, _i]
    lib.lt_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.lt_prefill_varlen.argtypes = [_vp, _vp, _vp, _i, _vp, _i, _ll, _vp, _vp, _i,
                                      _vp, _vp, _i, _i, _i, _vp]
    lib.lt_prefill_varlen.restype = _i
    lib.lt_decode.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _i, _vp]
    lib.lt_decode.restype = _i
    lib.lt_prefill_norm_gate.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _f, _vp, _i, _vp, _vp,
                                         _i, _ll, _i, _i, _i, _vp, ctypes.c_size_t, _vp]
    lib.lt_prefill_norm_gate.restype = _i
    lib.lt_prefill_varlen_norm_gate.argtypes = [_vp, _vp, _vp, _i, _vp, _i, _ll, _vp, _vp, _vp, _f,
                                                _vp, _i, _vp, _vp, _i, _i, _i, _vp]
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


def _dev_ptr(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def lt_prefill_workspace_bytes(batch, seqlen, heads, head_dim=HEAD_DIM, in_dtype=LT_BF16) -> int:
    return int(lib.lt_prefill_workspace_bytes(int(batch), int(seqlen), int(heads), int(head_dim),
                                              int(in_dtype)))


def lt_prefill(q, k, v, slopes, block, state_in=None, *, o=None, state_out=None,
               want_state=True, out_dtype=None, workspace=None, stream=None):
    """Fixed-length prefill. q, k, v: [batch, L, H, 128]; slopes: fp32 [H].

    Returns (o [batch, L, H, 128], state_out [batch, H, 128, 128] fp32 or None).
    ``state_out`` may be given (it may be ``state_in`` itself for an in-place
    update); otherwise one is allocated when ``want_state``. ``workspace`` is a
    uint8 device tensor of at least ``lt_prefill_workspace_bytes`` bytes; one
    is allocated when it is None and the plan wants one.
    """
    torch = _torch()
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [batch, L, H, d] shape")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    batch, L, H, d = q.shape
    out_dtype = out_dtype or torch.float32
    if o is None:
        o = torch.empty((batch, L, H, d), device=q.device, dtype=out_dtype)
    if state_out is None and want_state:
        state_out = torch.empty((batch, H, d, d), device=q.device, dtype=torch.float32)
    if workspace is None:
        nbytes = lt_prefill_workspace_bytes(batch, L, H, d, _dtype_code(q.dtype))
        if nbytes:
            workspace = torch.empty(nbytes, device=q.device, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.lt_prefill(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dtype_code(q.dtype),
                        _dev_ptr(slopes, "slopes"), _dev_ptr(o, "o"), _dtype_code(o.dtype),
                        _dev_ptr(state_in, "state_in"), _dev_ptr(state_out, "state_out"),
                        batch, L, H, d, int(block), _dev_ptr(workspace, "workspace"), ws_bytes,
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
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [batch, L, H, d] shape")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    batch, L, H, d = q.shape
    out_dtype = out_dtype or torch.float32
    if o is None:
        o = torch.empty((batch, L, H, d), device=q.device, dtype=out_dtype)
    if state_out is None and want_state:
        state_out = torch.empty((batch, H, d, d), device=q.device, dtype=torch.float32)
    st = lib.lt_prefill_noalloc(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                _dtype_code(q.dtype), _dev_ptr(slopes, "slopes"), _dev_ptr(o, "o"),
                                _dtype_code(o.dtype), _dev_ptr(state_in, "state_in"),
                                _dev_ptr(state_out, "state_out"), batch, L, H, d, int(block),
                                _stream(stream, q.device))
    _check(st, "lt_prefill_noalloc")
    return o, state_out


def lt_prefill_varlen(q, k, v, cu_seqlens, slopes, block, state_in=None, *, o=None,
                      state_out=None, want_state=True, out_dtype=None, stream=None):
    """Packed variable-length prefill. q, k, v: [T, H, 128]; cu_seqlens: int32 [n+1] on device.

    Returns (o [T, H, 128], state_out [n, H, 128, 128] fp32 or None).
    """
    torch = _torch()
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [T, H, d] shape")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    T, H, d = q.shape
    n = cu_seqlens.numel() - 1
    out_dtype = out_dtype or torch.float32
    if o is None:
        o = torch.empty((T, H, d), device=q.device, dtype=out_dtype)
    if state_out is None and want_state:
        state_out = torch.empty((n, H, d, d), device=q.device, dtype=torch.float32)
    st = lib.lt_prefill_varlen(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                               _dtype_code(q.dtype), _dev_ptr(cu_seqlens, "cu_seqlens"), n, T,
                               _dev_ptr(slopes, "slopes"), _dev_ptr(o, "o"), _dtype_code(o.dtype),
                               _dev_ptr(state_in, "state_in"), _dev_ptr(state_out, "state_out"),
                               H, d, int(block), _stream(stream, q.device))
    _check(st, "lt_prefill_varlen")
    return o, state_out


def lt_decode(q, k, v, slopes, state, *, o=None, out_dtype=None, stream=None):
    """One decode step. q, k, v: [batch, H, 128]; state: [batch, H, 128, 128] fp32, updated in place.

    Returns o [batch, H, 128].
    """
    torch = _torch()
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [batch, H, d] shape")
    batch, H, d = q.shape
    if state.dtype != torch.float32 or tuple(state.shape) != (batch, H, d, d):
        raise ValueError("state must be float32 [batch, H, d, d]")
    out_dtype = out_dtype or torch.float32
    if o is None:
        o = torch.empty((batch, H, d), device=q.device, dtype=out_dtype)
    st = lib.lt_decode(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dtype_code(q.dtype),
                       _dev_ptr(slopes, "slopes"), _dev_ptr(state, "state"), _dev_ptr(o, "o"),
                       _dtype_code(o.dtype), batch, H, d, _stream(stream, q.device))
    _check(st, "lt_decode")
    return o


def _check_gate(gate, like, norm_weight, heads):
    torch = _torch()
    if tuple(gate.shape) != tuple(like.shape) or gate.dtype != like.dtype:
        raise ValueError("gate must have the shape and dtype of q")
    if norm_weight.dtype != torch.float32 or tuple(norm_weight.shape) != (heads, HEAD_DIM):
        raise ValueError("norm_weight must be float32 [heads, 128]")


def lt_prefill_norm_gate(q, k, v, slopes, gate, norm_weight, eps, block, state_in=None, *, y=None,
                         state_out=None, want_state=True, out_dtype=None, workspace=None,
                         stream=None):
    """Fixed-length prefill followed by y = rmsnorm(o) * norm_weight * sigmoid(gate) per
    (token, head). q, k, v, gate: bf16 [batch, L, H, 128]; norm_weight: fp32 [H, 128].

    Returns (y [batch, L, H, 128], state_out or None); other arguments as lt_prefill.
    """
    torch = _torch()
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [batch, L, H, d] shape")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    batch, L, H, d = q.shape
    _check_gate(gate, q, norm_weight, H)
    out_dtype = out_dtype or torch.float32
    if y is None:
        y = torch.empty((batch, L, H, d), device=q.device, dtype=out_dtype)
    if state_out is None and want_state:
        state_out = torch.empty((batch, H, d, d), device=q.device, dtype=torch.float32)
    if workspace is None:
        nbytes = lt_prefill_workspace_bytes(batch, L, H, d, _dtype_code(q.dtype))
        if nbytes:
            workspace = torch.empty(nbytes, device=q.device, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.lt_prefill_norm_gate(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                  _dtype_code(q.dtype), _dev_ptr(slopes, "slopes"),
                                  _dev_ptr(gate, "gate"), _dev_ptr(norm_weight, "norm_weight"),
                                  float(eps), _dev_ptr(y, "y"), _dtype_code(y.dtype),
                                  _dev_ptr(state_in, "state_in"), _dev_ptr(state_out, "state_out"),
                                  batch, L, H, d, int(block), _dev_ptr(workspace, "workspace"),
                                  ws_bytes, _stream(stream, q.device))
    _check(st, "lt_prefill_norm_gate")
    return y, state_out


def lt_prefill_varlen_norm_gate(q, k, v, cu_seqlens, slopes, gate, norm_weight, eps, block,
                                state_in=None, *, y=None, state_out=None, want_state=True,
                                out_dtype=None, stream=None):
    """Packed variable-length prefill followed by the norm-gate epilogue.
    q, k, v, gate: bf16 [T, H, 128]; other arguments as lt_prefill_varlen.

    Returns (y [T, H, 128], state_out [n, H, 128, 128] or None).
    """
    torch = _torch()
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [T, H, d] shape")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    T, H, d = q.shape
    _check_gate(gate, q, norm_weight, H)
    n = cu_seqlens.numel() - 1
    out_dtype = out_dtype or torch.float32
    if y is None:
        y = torch.empty((T, H, d), device=q.device, dtype=out_dtype)
    if state_out is None and want_state:
        state_out = torch.empty((n, H, d, d), device=q.device, dtype=torch.float32)
    st = lib.lt_prefill_varlen_norm_gate(
        _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dtype_code(q.dtype),
        _dev_ptr(cu_seqlens, "cu_seqlens"), n, T, _dev_ptr(slopes, "slopes"),
        _dev_ptr(gate, "gate"), _dev_ptr(norm_weight, "norm_weight"), float(eps),
        _dev_ptr(y, "y"), _dtype_code(y.dtype), _dev_ptr(state_in, "state_in"),
        _dev_ptr(state_out, "state_out"), H, d, int(block), _stream(stream, q.device))
    _check(st, "lt_prefill_varlen_norm_gate")
    return y, state_out


def lt_decode_norm_gate(q, k, v, slopes, state, gate, norm_weight, eps, *, y=None, out_dtype=None,
                        stream=None):
    """One decode step followed by the norm-gate epilogue. q, k, v, gate: [batch, H, 128];
    state: [batch, H, 128, 128] fp32, updated in place. Returns y [batch, H, 128].
    """
    torch = _torch()
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [batch, H, d] shape")
    batch, H, d = q.shape
    _check_gate(gate, q, norm_weight, H)
    if state.dtype != torch.float32 or tuple(state.shape) != (batch, H, d, d):
        raise ValueError("state must be float32 [batch, H, d, d]")
    out_dtype = out_dtype or torch.float32
    if y is None:
        y = torch.empty((batch, H, d), device=q.device, dtype=out_dtype)
    st = lib.lt_decode_norm_gate(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                 _dtype_code(q.dtype), _dev_ptr(slopes, "slopes"),
                                 _dev_ptr(state, "state"), _dev_ptr(gate, "gate"),
                                 _dev_ptr(norm_weight, "norm_weight"), float(eps), _dev_ptr(y, "y"),
                                 _dtype_code(y.dtype), batch, H, d, _stream(stream, q.device))
    _check(st, "lt_decode_norm_gate")
    return y


def lt_decode_slots(q, k, v, slopes, state_pool, slot_ids, *, o=None, out_dtype=None, stream=None):
    """One decode step over a state pool. q, k, v: [batch, H, 128]; state_pool:
    [num_slots, H, 128, 128] fp32, updated in place; slot_ids: int32 [batch] on the
    device (out-of-range ids are padding rows with zero output). Returns o [batch, H, 128].
    """
    torch = _torch()
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [batch, H, d] shape")
    batch, H, d = q.shape
    if state_pool.dtype != torch.float32 or state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, d, d):
        raise ValueError("state_pool must be float32 [num_slots, H, d, d]")
    if slot_ids.dtype != torch.int32 or tuple(slot_ids.shape) != (batch,):
        raise ValueError("slot_ids must be int32 [batch]")
    out_dtype = out_dtype or torch.float32
    if o is None:
        o = torch.empty((batch, H, d), device=q.device, dtype=out_dtype)
    st = lib.lt_decode_slots(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dtype_code(q.dtype),
                             _dev_ptr(slopes, "slopes"), _dev_ptr(state_pool, "state_pool"),
                             int(state_pool.shape[0]), _dev_ptr(slot_ids, "slot_ids"), _dev_ptr(o, "o"),
                             _dtype_code(o.dtype), batch, H, d, _stream(stream, q.device))
    _check(st, "lt_decode_slots")
    return o


def lt_prefill_backward(q, k, v, dout, slopes, block, state_in=None, d_state_out=None, *, dq=None,
                        dk=None, dv=None, d_state_in=None, want_d_state_in=True, grad_dtype=None,
                        workspace=None, stream=None):
    """Gradients of sum(dout * o) + <d_state_out, S_final> for a fixed-length prefill.
    q, k, v, dout: bf16 [batch, L, H, 128]; state_in, d_state_out: fp32 [batch, H, 128, 128]
    or None. Returns (dq, dk, dv [batch, L, H, 128] in grad_dtype (default fp32),
    d_state_in [batch, H, 128, 128] fp32 or None).
    """
    torch = _torch()
    if q.dim() != 4 or any(x.shape != q.shape for x in (k, v, dout)):
        raise ValueError("q, k, v, dout must share one [batch, L, H, d] shape")
    if any(x.dtype != q.dtype for x in (k, v, dout)):
        raise TypeError("q, k, v, dout must share one dtype")
    batch, L, H, d = q.shape
    grad_dtype = grad_dtype or torch.float32
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
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.lt_prefill_backward(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                 _dev_ptr(dout, "dout"), _dtype_code(q.dtype),
                                 _dev_ptr(slopes, "slopes"), _dev_ptr(state_in, "state_in"),
                                 _dev_ptr(d_state_out, "d_state_out"), _dev_ptr(dq, "dq"),
                                 _dev_ptr(dk, "dk"), _dev_ptr(dv, "dv"), _dtype_code(dq.dtype),
                                 _dev_ptr(d_state_in, "d_state_in"), batch, L, H, d, int(block),
                                 _dev_ptr(workspace, "workspace"), ws_bytes, _stream(stream, q.device))
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
    if any(x.dtype != torch.bfloat16 for x in (q, k, v)):
        raise TypeError("q, k, v must be bfloat16")
    batch, L, Hq, d = q.shape
    Hkv = k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out_dtype = out_dtype or torch.float32
    if o is None:
        o = torch.empty((batch, L, Hq, d), device=q.device, dtype=out_dtype)
    if k_rope is None:
        k_rope = torch.empty_like(k)
    st = lib.lt_softmax_prefill(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(o, "o"),
                                _dtype_code(o.dtype), _dev_ptr(k_rope, "k_rope"), batch, L, Hq, Hkv, d,
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
    if any(x.dtype != torch.bfloat16 for x in (q, k_new, v_new, k_cache, v_cache)):
        raise TypeError("q, k_new, v_new and the caches must be bfloat16")
    if lengths.dtype != torch.int32 or tuple(lengths.shape) != (batch,):
        raise ValueError("lengths must be int32 [batch]")
    cap = k_cache.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out_dtype = out_dtype or torch.float32
    if o is None:
        o = torch.empty((batch, Hq, d), device=q.device, dtype=out_dtype)
    if workspace is None:
        nb = lt_softmax_decode_workspace_bytes(batch, cap, Hq, Hkv, d)
        workspace = torch.empty(max(nb, 1), device=q.device, dtype=torch.uint8) if nb else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.lt_softmax_decode(_dev_ptr(q, "q"), _dev_ptr(k_new, "k_new"), _dev_ptr(v_new, "v_new"),
                               _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
                               _dev_ptr(lengths, "lengths"), _dev_ptr(o, "o"), _dtype_code(o.dtype), batch,
                               cap, Hq, Hkv, d, int(rope_dims), float(rope_base), scale,
                               _dev_ptr(workspace, "workspace"), wbytes, _stream(stream, q.device))
    _check(st, "lt_softmax_decode")
    return o
