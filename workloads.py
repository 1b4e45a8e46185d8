"""Seeded synthetic inputs for the Lightning Attention workloads.

This module only draws random numbers and lays them out; it holds none of the
operator's arithmetic. Both the oracle side and the HIP side of every test and
of the benchmark take their inputs from here, so the two see identical values.

Shapes follow the MiniMax-M1 Lightning layer: 64 heads of dimension 128
(MiniMax Signal Lab · M1, §02 architecture card "Attention Projection 64 heads
x 128", and §04 Context Cache, whose 293.6 MB fixed FP32 state for 70 layers is
exactly 70 x 64 x 128 x 128 x 4 bytes). The pages give no slope values; the
workloads use s_h = 2^(-8 (h+1) / H).

Recipe (stated once more in the design doc):
  * q, k, v ~ N(0, 1) / sqrt(128), drawn in fp32, then rounded to bf16 with
    round-to-nearest-even where the workload is bf16. The oracle consumes the
    rounded values, so input quantisation never counts as kernel error.
  * carried-in states ~ N(0, 0.01) read as variance 0.01 (std 0.1), fp32.
  * varlen lengths: 16 integers uniform on [1024, 65536], packed by cu_seqlens.
  * softmax layers (the hybrid's other attention type, §02: 64 query heads,
    8 K/V heads of 128, RoPE on 64 dims): q, k, v ~ N(0, std^2), std 1 by
    default so the scaled scores are O(1) like real attention logits, rounded
    to bf16; RoPE base 10000 (the pages give none).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 128
INPUT_SCALE = 1.0 / math.sqrt(128.0)


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    heads: int
    head_dim: int
    block: int
    dtype: str  # "f32" or "bf16" (input dtype); outputs and states are fp32
    seed: int
    extra: dict = field(default_factory=dict)


TINY_F32 = Workload("tiny_f32_prefill", 1, 1024, 8, 128, 64, "f32", 1001)
M1_LAYER = Workload("m1_layer_bf16_prefill", 1, 32768, 64, 128, 256, "bf16", 1002)
LONG_1M = Workload("long_context_1m_bf16_prefill", 1, 1 << 20, 64, 128, 256, "bf16", 1003)
DECODE = Workload("batched_decode", 256, 1, 64, 128, 0, "bf16", 1004,
                  {"steps": 1000, "history": 4096})
VARLEN = Workload("varlen_carried_state_prefill", 16, 0, 64, 128, 256, "bf16", 1005,
                  {"min_len": 1024, "max_len": 65536})

SOFTMAX_PREFILL = Workload("m1_softmax_layer_bf16_prefill", 1, 32768, 64, 128, 0, "bf16", 1006,
                           {"kv_heads": 8, "rope_dims": 64, "rope_base": 10000.0})
SOFTMAX_DECODE = Workload("m1_softmax_layer_bf16_decode", 16, 1, 64, 128, 0, "bf16", 1007,
                          {"kv_heads": 8, "rope_dims": 64, "rope_base": 10000.0, "context": 32768})

ALL = [TINY_F32, M1_LAYER, LONG_1M, DECODE, VARLEN, SOFTMAX_PREFILL, SOFTMAX_DECODE]


def slopes(heads: int) -> np.ndarray:
    """Per-head decay slopes s_h = 2^(-8 (h+1) / H) as fp32."""
    return np.array([2.0 ** (-8.0 * (h + 1) / heads) for h in range(heads)],
                    dtype=np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32 holding them."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    out = rounded.view(np.float32).copy()
    nan = np.isnan(x)
    out[nan] = x[nan]
    return out


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def qkv_host(seed: int, shape, dtype: str = "bf16"):
    """q, k, v as fp32 NumPy arrays holding values of the given input dtype."""
    g = rng(seed)
    out = []
    for _ in range(3):
        x = (g.standard_normal(shape, dtype=np.float32) * np.float32(INPUT_SCALE))
        out.append(round_bf16(x) if dtype == "bf16" else x.astype(np.float32))
    return tuple(out)


def state_host(seed: int, shape, std: float = 0.1) -> np.ndarray:
    """Random fp32 carried-in states, N(0, std^2)."""
    g = rng(seed)
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def varlen_lengths(seed: int, n: int = 16, lo: int = 1024, hi: int = 65536) -> np.ndarray:
    """n sequence lengths uniform on the integers [lo, hi]."""
    return rng(seed).integers(lo, hi, size=n, endpoint=True).astype(np.int64)


def cu_seqlens(lengths) -> np.ndarray:
    """Exclusive prefix sum [0, l0, l0+l1, ...] as int32."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    assert cu[-1] < 2 ** 31
    return cu.astype(np.int32)


def qkv_device(seed: int, shape, dtype: str = "bf16", device="cuda"):
    """q, k, v drawn on the device with a seeded torch generator.

    fp32 N(0,1)/sqrt(128), then rounded to bf16 (torch's conversion rounds to
    nearest even) for bf16 workloads. Used for the large workloads whose host
    generation would be slow; the oracle reads these same values back.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = []
    for _ in range(3):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        x.mul_(INPUT_SCALE)
        out.append(x.to(torch.bfloat16) if dtype == "bf16" else x)
    return tuple(out)


def state_device(seed: int, shape, std: float = 0.1, device="cuda"):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.mul_(std)


# Inputs of the norm-gate epilogue (normalisation and gate after the sum): gate
# pre-activations N(0, 1) in the input dtype, weights U[0.5, 1.5] fp32 [H, d],
# eps 1e-6.
NORM_EPS = 1e-6


def gate_host(seed: int, shape, dtype: str = "bf16") -> np.ndarray:
    x = rng(seed).standard_normal(shape, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def norm_weight_host(seed: int, heads: int, d: int = HEAD_DIM) -> np.ndarray:
    return rng(seed).uniform(0.5, 1.5, (heads, d)).astype(np.float32)


def gate_device(seed: int, shape, dtype: str = "bf16", device="cuda"):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def softmax_qkv_host(seed: int, batch: int, seqlen: int, q_heads: int, kv_heads: int,
                     d: int = HEAD_DIM, std: float = 1.0):
    """q [batch, L, Hq, d], k, v [batch, L, Hkv, d]: N(0, std^2) rounded to bf16
    (fp32 arrays holding bf16 values)."""
    g = rng(seed)
    shapes = [(batch, seqlen, q_heads, d), (batch, seqlen, kv_heads, d), (batch, seqlen, kv_heads, d)]
    return tuple(round_bf16(g.standard_normal(sh, dtype=np.float32) * np.float32(std)) for sh in shapes)


def softmax_qkv_device(seed: int, batch: int, seqlen: int, q_heads: int, kv_heads: int,
                       d: int = HEAD_DIM, std: float = 1.0, device="cuda"):
    """Device-drawn softmax-layer inputs (bf16 tensors) for the large workloads."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    shapes = [(batch, seqlen, q_heads, d), (batch, seqlen, kv_heads, d), (batch, seqlen, kv_heads, d)]
    return tuple((torch.randn(sh, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)
                 for sh in shapes)
