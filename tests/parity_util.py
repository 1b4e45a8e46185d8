"""Helpers shared by the GPU parity tests (no test functions here).

Every GPU-vs-oracle comparison goes through :func:`parity_err`, which holds a
(sequence, head) slice to two bounds at once:

  * the per-head bound: relative L2 error ||x - y|| / ||y|| over the whole
    slice (y = oracle), <= tol (1e-5 for fp32 inputs, 1e-2 for bf16 inputs);
  * a per-row bound: for every row t of the slice (one token's d outputs, or
    one key row of a d x d state), ||x_t - y_t|| <= ROW_FACTOR * tol * rms(y),
    where rms(y) = sqrt(mean_t ||y_t||^2) is the slice's RMS row norm (so rows
    that are small only because early tokens have little history do not set
    the bound).

``parity_err`` returns max(relative L2, worst row ratio / ROW_FACTOR), so
``parity_err(x, y) <= tol`` holds exactly when both bounds do. The per-head
bound alone cannot see a few wrong rows in a long sequence: at L = 32768 one
entirely wrong row adds only sqrt(1/32768) ~ 0.0055 to it. The row bound
catches such a row (its ratio is ~1, against 5e-2 for bf16), including the
rows where a segmented plan could go wrong (segment starts, the cuts between
warm-up ranges, sub-block edges, the last token), since every row of every
compared slice is checked.

ROW_FACTOR = 5: with bf16 inputs the per-row error of a correct kernel is the
rounding of its bf16 operands (the scores and the state, 2^-9 relative),
about 2e-3 of a typical row norm, with rows near the head's RMS norm; the
worst row over 2^20 tokens stays within a small multiple of that, well under
5e-2, while a wrong row sits near 1.
"""

from __future__ import annotations

import numpy as np

# Tolerances on relative L2 error per (sequence, head), for O and final state.
TOL_F32 = 1e-5
TOL_BF16 = 1e-2
# Row bound = ROW_FACTOR * (per-head tolerance) * (RMS row norm of the slice).
ROW_FACTOR = 5.0

def source_hash() -> str:
    """The library's source hash as the build bakes it in (see linear_attention_amd.build)."""
    from linear_attention_amd import build as b

    return b.source_hash()


def ensure_built():
    """Build liblightning.so when it is missing or was built from other sources
    than the tree's (its lt_build_id differs from the hash of csrc/ and include/)."""
    from linear_attention_amd import build as b

    if not b.library_is_current():
        b.build()


def slice_errors(x, y):
    """(relative L2, worst row ratio, index of that row) of a slice in fp64.

    x, y: [..., rows, d] (leading dims flattened into rows); a 1-D vector is
    one row. The row ratio is ||x_t - y_t|| / rms_t ||y_t||. A zero oracle
    slice compares absolutely. Non-finite values anywhere give inf."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    if x.shape != y.shape:
        raise AssertionError(f"shape mismatch {x.shape} vs {y.shape}")
    if x.ndim == 1:
        x = x[None]
        y = y[None]
    x = x.reshape(-1, x.shape[-1])
    y = y.reshape(-1, y.shape[-1])
    if not (np.isfinite(x).all() and np.isfinite(y).all()):
        return float("inf"), float("inf"), -1
    dr = np.sqrt(np.sum((x - y) ** 2, axis=1))
    yr2 = np.sum(y * y, axis=1)
    ny = float(np.sqrt(yr2.sum()))
    rel = float(np.sqrt((dr * dr).sum()) / ny) if ny > 0 else float(np.sqrt((dr * dr).sum()))
    rms = float(np.sqrt(yr2.mean()))
    ratios = dr / rms if rms > 0 else dr
    i = int(np.argmax(ratios))
    return rel, float(ratios[i]), i


def parity_err(x, y) -> float:
    """max(relative L2, worst row ratio / ROW_FACTOR) of a slice against the
    oracle y: <= tol iff the per-head bound and every row's bound hold."""
    rel, row, _ = slice_errors(x, y)
    return max(rel, row / ROW_FACTOR)


def rel_l2(x, y) -> float:
    """Plain ||x - y||_2 / ||y||_2 in fp64 (y is the reference); 0-norm y compares
    absolutely. For GPU-vs-oracle comparisons use :func:`parity_err`."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    ny = np.linalg.norm(y)
    err = np.linalg.norm(x - y)
    return float(err / ny) if ny > 0 else float(err)


def max_rel_per_head(o_gpu, o_ref, cu):
    """Worst parity_err over (sequence, head) slices of packed outputs [T, H, d]."""
    worst = 0.0
    for a, b in zip(cu[:-1], cu[1:]):
        if b <= a:
            continue
        for h in range(o_ref.shape[1]):
            worst = max(worst, parity_err(o_gpu[a:b, h], o_ref[a:b, h]))
    return worst


def max_rel_states(s_gpu, s_ref):
    """Worst parity_err over [units, H, d, d] states (rows = key index)."""
    worst = 0.0
    for n in range(s_ref.shape[0]):
        for h in range(s_ref.shape[1]):
            worst = max(worst, parity_err(s_gpu[n, h], s_ref[n, h]))
    return worst


# ---------------------------------------------------------------------------
# Rows where a segmented plan can go wrong, listed explicitly. The launch plan
# of lt_prefill (batch-1 style calls with fewer than 256 (sequence, head) pairs
# and at least 4096 tokens per sequence): G = ceil(256 / (batch * heads))
# segments, at most L / 2048, of seg = ceil(L / G) tokens rounded up to a
# multiple of 128. A head with slope s whose warm-up W = 128 * floor((floor(16 /
# (s log2 e)) + 128) / 128) is shorter than a segment takes warm-up ranges
# (cut at multiples of 128 tokens, each rebuilding its carried-in state from
# the W tokens before it); the others take the pre-pass. The backward's reverse
# pass does the same counted from the end of the sequence.

LOG2E = 1.4426950408889634


def plan_segments(batch, L, heads):
    """(segments, seg_len) of a fixed-length bf16 lt_prefill with a workspace."""
    uh = batch * heads
    if uh >= 256:
        return 1, L
    g = (256 + uh - 1) // uh
    g = min(g, L // 2048)
    if g < 2:
        return 1, L
    seg = (L + g - 1) // g
    seg = (seg + 127) // 128 * 128
    g = (L + seg - 1) // seg
    return (g, seg) if g >= 2 else (1, L)


def boundary_rows(L, seg_len, segments, slope):
    """Rows (token indices) next to every place a segmented plan switches: segment
    starts +-2 (heads on the pre-pass), every 64-token sub-block edge +-1 (the
    cuts between the warm-up ranges of the other heads fall on such edges), and
    the last token. ``slope`` is kept for the callers; the rows do not depend
    on it."""
    del slope
    rows = {0, L - 1}
    for c in range(0, L, 64):
        rows.update((c - 1, c))
    for g in range(segments):
        s0 = g * seg_len
        rows.update(range(s0 - 2, s0 + 3))
    return sorted(r for r in rows if 0 <= r < L)


def boundary_row_err(x, y, rows) -> float:
    """Worst row ratio / ROW_FACTOR over the listed rows of an [L, d] slice (the
    RMS is that of the whole slice), comparable with the per-head tolerance."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    rms = float(np.sqrt(np.mean(np.sum(y * y, axis=1))))
    idx = np.asarray(rows, np.int64)
    d = np.sqrt(np.sum((x[idx] - y[idx]) ** 2, axis=1))
    return float(d.max() / rms / ROW_FACTOR) if len(idx) else 0.0


def to_host_f32(t) -> np.ndarray:
    import torch

    return t.detach().to(torch.float32).cpu().numpy()


def to_device(x: np.ndarray, dtype: str, device="cuda"):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def segment_boundary_err(x, y, batch, L, heads, slope) -> float:
    """boundary_row_err of one (sequence, head) slice [L, d] over the rows next to
    the switches of the plan lt_prefill uses for a [batch, L, heads] call."""
    g, seg = plan_segments(batch, L, heads)
    return boundary_row_err(x, y, boundary_rows(L, seg, g, slope))
