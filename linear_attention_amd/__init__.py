"""Lightning Attention for MI355X (gfx950): HIP kernels behind a C ABI.

The operator (MiniMax Signal Lab · M1, §03 Lightning Attention) is causal
linear attention with a per-head exponential decay, evaluated block by block
with a fixed d x d fp32 state per head, plus its one-token decode step.

``lt_init`` (optional: loads the GPU code before the first call),
``lt_prefill``, ``lt_prefill_noalloc`` (the same with the library's static
scratch, for callers that cannot allocate), ``lt_prefill_workspace_bytes``,
``lt_prefill_varlen``,
``lt_decode``, ``lt_decode_slots`` (decode over a state pool),
``lt_prefill_backward`` (gradients of a prefill) and the ``*_norm_gate``
variants (the operator followed by the
normalisation and gate of the §03 data-flow figure) mirror the C entry points
of ``include/lightning.h`` one to one, as do ``lt_softmax_prefill`` and
``lt_softmax_decode`` (the hybrid's other layer type: causal softmax attention
with grouped K/V heads and partial RoPE, §02 of the same pages, and its decode
step over a KV cache).
The shared library is loaded on first use of any of these names (so the build
module can be imported before the library exists); a missing library raises
ImportError there, and there is no fallback path.
"""

_NATIVE_NAMES = (
    "lt_init", "lt_prefill", "lt_prefill_noalloc", "lt_prefill_workspace_bytes", "lt_prefill_varlen",
    "lt_prefill_varlen_workspace_bytes", "lt_decode",
    "lt_prefill_norm_gate", "lt_prefill_varlen_norm_gate", "lt_decode_norm_gate", "lt_decode_slots",
    "lt_prefill_backward", "lt_softmax_prefill", "lt_softmax_decode", "lt_softmax_decode_workspace_bytes",
    "LightningError", "lib", "status_string", "EXPORTS", "LIB_PATH", "HEAD_DIM", "LT_OK",
    "LT_ERR_NULL", "LT_ERR_SHAPE", "LT_ERR_BLOCK", "LT_ERR_DTYPE", "LT_ERR_ALIAS", "LT_ERR_HIP",
    "LT_ERR_VALUE", "LT_ERR_SCRATCH",
    "LT_F32", "LT_BF16", "LT_MAX_BLOCK",
)

__all__ = list(_NATIVE_NAMES)


def __getattr__(name):
    if name in _NATIVE_NAMES:
        from . import _native

        return getattr(_native, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
