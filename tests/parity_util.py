"""Helpers shared by the GPU parity tests (no test functions here)."""

from __future__ import annotations

import os

import numpy as np

# Tolerances on relative L2 error per (sequence, head), for O and final state.
TOL_F32 = 1e-5
TOL_BF16 = 1e-2


def ensure_built():
    """Build liblightning.so if it is missing (never rebuilds an existing one)."""
    from linear_attention_amd import build as b

    if not os.path.exists(b.LIB):
        b.build()


def rel_l2(x, y) -> float:
    """||x - y||_2 / ||y||_2 in fp64 (y is the oracle); 0-norm y compares absolutely."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    ny = np.linalg.norm(y)
    err = np.linalg.norm(x - y)
    return float(err / ny) if ny > 0 else float(err)


def max_rel_per_head(o_gpu, o_ref, cu, head_axis=1):
    """Worst relative L2 over (sequence, head) slices of packed outputs [T, H, d]."""
    worst = 0.0
    for a, b in zip(cu[:-1], cu[1:]):
        if b <= a:
            continue
        for h in range(o_ref.shape[head_axis]):
            worst = max(worst, rel_l2(o_gpu[a:b, h], o_ref[a:b, h]))
    return worst


def max_rel_states(s_gpu, s_ref):
    """Worst relative L2 over [units, H, d, d] states."""
    worst = 0.0
    for n in range(s_ref.shape[0]):
        for h in range(s_ref.shape[1]):
            worst = max(worst, rel_l2(s_gpu[n, h], s_ref[n, h]))
    return worst


def to_host_f32(t) -> np.ndarray:
    import torch

    return t.detach().to(torch.float32).cpu().numpy()


def to_device(x: np.ndarray, dtype: str, device="cuda"):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    return t.to(torch.bfloat16) if dtype == "bf16" else t
