"""Lightning Attention oracle: plain, slow, fp64 CPU reference.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package. The HIP product
path (``linear_attention_amd``) never imports it and shares no code with it.

Three independent formulations of the same operator, all in fp64:

``recurrence*``
    The per-token recurrence ``S <- e^{-s} S + k^T v ; o = q S`` (compiled C,
    ``lightning_oracle.c``), which is what the block form of MiniMax Signal
    Lab · M1, §03 Lightning Attention, reduces to with a one-token block, and
    the "cumsum" that the fishai commentary on M1 says the block split avoids.
    This is the oracle the GPU path is checked against.
``brute_force``
    The quadratic masked form: the §03 intra-block formula
    ``[(Q K^T) ⊙ D] V`` with one block spanning the whole sequence, plus the
    decayed read of the carried-in state (a one-block ``O_inter``).
``block_form``
    The §03 block decomposition itself, step by step in the pages' notation
    (``D``, ``d_q``, ``d_k``, block decay, last short block of length ``m``).
``backward*``
    Gradients of ``sum(dO * O) + <dS, S_final>`` with respect to q, k, v and
    S0: the reverse-mode derivative of the per-token recurrence (compiled C;
    the pages give no backward).
``softmax_attention`` / ``softmax_decode``
    The hybrid's other attention type (MiniMax Signal Lab · M1, §02: 64 query
    heads of 128, K/V 8 x 128, RoPE on 64 of 128 dims in the softmax layers
    only): causal softmax attention with grouped K/V heads and partial
    rotary position embedding, and its one-token decode over a KV cache.
``decode_slots``
    One decode step over a pool of per-sequence states addressed by slot ids
    (concurrent sequences, each with the fixed-size state of §04).
``norm_gate``
    The step after the operator in the §03 data-flow figure: the summed output
    is normalised and gated (RMS normalisation per (token, head), a weight per
    (head, feature), a logistic-sigmoid gate; the pages name neither form).

Readings of points the pages leave open:
positions inside a block are 1-indexed, ``d_q[i] = e^{-s i}``,
``d_k[j] = e^{-s (m - j)}``, the state decays by ``e^{-s m}`` per block of
``m`` tokens, ``D`` includes the diagonal, ``⊙`` with a length-``m`` vector
scales token rows, and the operator output is ``O_intra + O_inter`` with no
normaliser. A carried-in state ``S0`` is decayed by the first token.

Parity status: pinned (see ``tests/test_oracle.py``).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lightning_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblightning_oracle.so")

# gcc flags: portable x86-64-v3 so the library built here also runs on the GPU
# host; IEEE fp64 (no fast-math).
GCC_CMD = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-shared", "-fPIC",
           "-Wall", "-Wextra", _SRC, "-o", _LIB_PATH]


def build() -> str:
    """Compile the C oracle in place and return the library path."""
    subprocess.run(GCC_CMD, check=True)
    return _LIB_PATH


class _Unit(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("in_stride", ctypes.c_longlong),
        ("len", ctypes.c_longlong),
        ("slope", ctypes.c_double),
        ("s0", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("o_stride", ctypes.c_longlong),
        ("s_final", ctypes.c_void_p),
    ]


class _BwdUnit(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("dout", ctypes.c_void_p),
        ("in_stride", ctypes.c_longlong),
        ("len", ctypes.c_longlong),
        ("slope", ctypes.c_double),
        ("s0", ctypes.c_void_p),
        ("ds", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("o_stride", ctypes.c_longlong),
        ("ds0", ctypes.c_void_p),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if (not os.path.exists(_LIB_PATH)
                or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.lto_recurrence.argtypes = [ctypes.POINTER(_Unit), ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int]
        lib.lto_recurrence.restype = ctypes.c_int
        lib.lto_backward.argtypes = [ctypes.POINTER(_BwdUnit), ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int]
        lib.lto_backward.restype = ctypes.c_int
        lib.lto_max_threads.argtypes = []
        lib.lto_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    """Threads the C oracle's OpenMP region uses by default."""
    return int(_load().lto_max_threads())


def _f32(x):
    return np.ascontiguousarray(np.asarray(x), dtype=np.float32)


def recurrence_packed(q, k, v, slopes, cu_seqlens, s0=None, heads=None,
                      want_o=True, threads=0):
    """Per-token recurrence over packed sequences, every (sequence, head) unit.

    q, k, v: [T, H, d] values (cast to float32; bf16/fp32 inputs are exact).
    slopes: [H] fp32 slopes (widened to fp64).
    cu_seqlens: [n+1] sequence boundaries, cu[0] = 0, cu[n] = T.
    s0: [n, H, d, d] carried-in states or None (zero).
    heads: optional list of head indices to compute (default: all).
    Returns (o [T, len(heads), d] fp64 or None, s_final [n, len(heads), d, d] fp64).
    """
    q, k, v = _f32(q), _f32(k), _f32(v)
    T, H, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    slopes = np.asarray(slopes, dtype=np.float32)
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    n = len(cu) - 1
    assert cu[0] == 0 and cu[-1] == T and all(b >= a for a, b in zip(cu, cu[1:]))
    hs = list(range(H)) if heads is None else [int(h) for h in heads]
    nh = len(hs)
    if s0 is not None:
        s0 = np.ascontiguousarray(s0, dtype=np.float64)
        assert s0.shape == (n, H, d, d)
    o = np.zeros((T, nh, d), dtype=np.float64) if want_o else None
    sf = np.zeros((n, nh, d, d), dtype=np.float64)

    units = (_Unit * (n * nh))()
    f4, f8 = 4, 8
    idx = 0
    for si in range(n):
        a, b = cu[si], cu[si + 1]
        for hj, h in enumerate(hs):
            u = units[idx]
            base = (a * H + h) * d * f4
            u.q = q.ctypes.data + base
            u.k = k.ctypes.data + base
            u.v = v.ctypes.data + base
            u.in_stride = H * d
            u.len = b - a
            u.slope = float(slopes[h])
            u.s0 = (s0.ctypes.data + ((si * H + h) * d * d) * f8) if s0 is not None else None
            if want_o:
                u.o = o.ctypes.data + ((a * nh + hj) * d) * f8
                u.o_stride = nh * d
            else:
                u.o = None
                u.o_stride = 0
            u.s_final = sf.ctypes.data + ((si * nh + hj) * d * d) * f8
            idx += 1
    rc = _load().lto_recurrence(units, n * nh, d, int(threads))
    if rc != 0:
        raise RuntimeError("oracle recurrence failed")
    return o, sf


def recurrence_batch(q, k, v, slopes, s0=None, heads=None, want_o=True, threads=0):
    """Per-token recurrence for a fixed-length batch.

    q, k, v: [batch, L, H, d]; s0: [batch, H, d, d] or None.
    Returns (o [batch, L, len(heads), d] or None, s_final [batch, len(heads), d, d]).
    """
    q = _f32(q)
    bsz, L, H, d = q.shape
    cu = np.arange(bsz + 1) * L
    o, sf = recurrence_packed(q.reshape(bsz * L, H, d), _f32(k).reshape(bsz * L, H, d),
                              _f32(v).reshape(bsz * L, H, d), slopes, cu, s0=s0,
                              heads=heads, want_o=want_o, threads=threads)
    if o is not None:
        o = o.reshape(bsz, L, o.shape[1], d)
    return o, sf


def recurrence(q, k, v, s, s0=None, want_o=True):
    """Per-token recurrence for one (sequence, head) unit: q, k, v [L, d]."""
    q = _f32(q)
    L, d = q.shape
    s0b = None if s0 is None else np.asarray(s0, dtype=np.float64).reshape(1, 1, d, d)
    o, sf = recurrence_packed(q.reshape(L, 1, d), _f32(k).reshape(L, 1, d),
                              _f32(v).reshape(L, 1, d), np.array([s], np.float32),
                              [0, L], s0=s0b, want_o=want_o)
    return (None if o is None else o.reshape(L, d)), sf.reshape(d, d)


def decode(q, k, v, slopes, state):
    """One decode step for every (sequence, head): one iteration of the recurrence.

    q, k, v: [batch, H, d]; state: [batch, H, d, d] (fp64 copy is made).
    Returns (o [batch, H, d] fp64, new_state [batch, H, d, d] fp64).
    """
    q, k, v = _f32(q), _f32(k), _f32(v)
    bsz, H, d = q.shape
    st = np.ascontiguousarray(state, dtype=np.float64).reshape(bsz, H, d, d)
    cu = np.arange(bsz + 1)
    o, sf = recurrence_packed(q.reshape(bsz, H, d), k, v, slopes, cu, s0=st)
    return o.reshape(bsz, H, d), sf


def recurrence_loop(q, k, v, s, s0=None):
    """Pure NumPy per-token loop for one unit (small cases; same definition as the C code)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    L, d = q.shape
    lam = np.exp(-np.float64(np.float32(s)))
    S = np.zeros((d, d)) if s0 is None else np.array(s0, np.float64)
    o = np.zeros((L, d))
    for i in range(L):
        S = lam * S + np.outer(k[i], v[i])
        o[i] = q[i] @ S
    return o, S


def brute_force(q, k, v, s, s0=None):
    """Quadratic masked form for one unit: one block spanning all L tokens.

    o_i = sum_{j<=i} e^{-s(i-j)} (q_i . k_j) v_j + e^{-s i} q_i S0,
    S_L = sum_j e^{-s(L-j)} k_j^T v_j + e^{-s L} S0   (positions 1..L).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    L, d = q.shape
    s = np.float64(np.float32(s))
    pos = np.arange(1, L + 1, dtype=np.float64)
    diff = pos[:, None] - pos[None, :]
    D = np.where(diff >= 0, np.exp(-s * np.maximum(diff, 0.0)), 0.0)
    o = ((q @ k.T) * D) @ v
    wk = np.exp(-s * (L - pos))
    S = (k * wk[:, None]).T @ v
    if s0 is not None:
        s0 = np.asarray(s0, np.float64)
        o = o + (q * np.exp(-s * pos)[:, None]) @ s0
        S = S + np.exp(-s * L) * s0
    return o, S


def block_form(q, k, v, s, block, s0=None):
    """The §03 block decomposition for one unit, in fp64, block length ``block``.

    For each block t of m tokens (m = block, or the remainder for the last one),
    with positions i, j = 1..m:
        D_ij   = e^{-s(i-j)} [i >= j]
        d_q[i] = e^{-s i},  d_k[j] = e^{-s(m-j)}
        O_t    = [(Q_t K_t^T) ⊙ D] V_t + (Q_t ⊙ d_q) S_{t-1}
        S_t    = e^{-s m} S_{t-1} + (K_t ⊙ d_k)^T V_t
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    L, d = q.shape
    s = np.float64(np.float32(s))
    S = np.zeros((d, d)) if s0 is None else np.array(s0, np.float64)
    o = np.zeros((L, d))
    for t0 in range(0, L, block):
        m = min(block, L - t0)
        Qt, Kt, Vt = q[t0:t0 + m], k[t0:t0 + m], v[t0:t0 + m]
        i = np.arange(1, m + 1, dtype=np.float64)
        diff = i[:, None] - i[None, :]
        D = np.where(diff >= 0, np.exp(-s * np.maximum(diff, 0.0)), 0.0)
        dq = np.exp(-s * i)
        dk = np.exp(-s * (m - i))
        o_intra = ((Qt @ Kt.T) * D) @ Vt
        o_inter = (Qt * dq[:, None]) @ S
        o[t0:t0 + m] = o_intra + o_inter
        S = np.exp(-s * m) * S + (Kt * dk[:, None]).T @ Vt
    return o, S


def norm_gate(o, gate, weight, eps):
    """Post-sum normalisation and gating, in fp64.

    MiniMax Signal Lab · M1, §03 (data-flow figure): after the intra- and
    inter-block outputs are added, the result passes through a normalisation
    and a gate. The pages name neither; the reading used here: each (token,
    head) vector of d features is divided by its root mean square,
    sqrt(mean(o^2) + eps), multiplied by a weight per (head, feature), and
    multiplied by the logistic sigmoid of a gate tensor of the same shape as o.

    o, gate: [..., H, d]; weight: [H, d]; eps >= 0. Returns fp64 [..., H, d].
    """
    o = np.asarray(o, np.float64)
    g = np.asarray(gate, np.float64)
    w = np.asarray(weight, np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return o / np.sqrt(ms + np.float64(eps)) * w * (1.0 / (1.0 + np.exp(-g)))


def decode_slots(q, k, v, slopes, pool, slot_ids):
    """One decode step of `batch` sequences whose states live in a pool.

    MiniMax Signal Lab · M1, §04: every concurrent sequence keeps its own
    fixed-size state (d x d fp32 per head), so a serving batch addresses a pool
    of such states. Sequence b reads and updates pool[slot_ids[b]] with one
    step of the recurrence; an id outside [0, num_slots) marks a padding row:
    its output is zero and the pool is untouched.

    q, k, v: [batch, H, d]; pool: [num_slots, H, d, d]; slot_ids: [batch] int.
    Returns (o [batch, H, d] fp64, new_pool [num_slots, H, d, d] fp64).
    """
    pool = np.array(pool, dtype=np.float64)
    ids = np.asarray(slot_ids, np.int64)
    bsz, H, d = np.shape(q)
    o = np.zeros((bsz, H, d))
    live = [b for b in range(bsz) if 0 <= ids[b] < pool.shape[0]]
    if live:
        sl = ids[live]
        ob, sb = decode(np.asarray(q)[live], np.asarray(k)[live], np.asarray(v)[live], slopes,
                        pool[sl])
        o[live] = ob
        pool[sl] = sb
    return o, pool


def backward_packed(q, k, v, dout, slopes, cu_seqlens, s0=None, ds=None, threads=0):
    """Gradients of the operator over packed sequences, every (sequence, head).

    The loss is l = sum_t dout_t . o_t + <ds, S_final> per (sequence, head);
    returns (dq, dk, dv [T, H, d] fp64, ds0 [n, H, d, d] fp64) with
      dq_t = dout_t S_t^T,  G_t = q_t^T dout_t + e^{-s} G_{t+1} (G_L adds ds),
      dk_t = G_t v_t,  dv_t = G_t^T k_t,  ds0 = e^{-s} G_1
    (reverse-mode derivative of the per-token recurrence; the pages give no
    backward). q, k, v, dout: [T, H, d] (read as float32); s0, ds: [n, H, d, d]
    or None (zero).
    """
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    T, H, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape and dout.shape == q.shape
    slopes = np.asarray(slopes, dtype=np.float32)
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    n = len(cu) - 1
    assert cu[0] == 0 and cu[-1] == T and all(b >= a for a, b in zip(cu, cu[1:]))
    if s0 is not None:
        s0 = np.ascontiguousarray(s0, dtype=np.float64)
        assert s0.shape == (n, H, d, d)
    if ds is not None:
        ds = np.ascontiguousarray(ds, dtype=np.float64)
        assert ds.shape == (n, H, d, d)
    dq, dk, dv = (np.zeros((T, H, d), dtype=np.float64) for _ in range(3))
    ds0 = np.zeros((n, H, d, d), dtype=np.float64)
    units = (_BwdUnit * (n * H))()
    f4, f8 = 4, 8
    idx = 0
    for si in range(n):
        a, b = cu[si], cu[si + 1]
        for h in range(H):
            u = units[idx]
            base = (a * H + h) * d * f4
            u.q, u.k, u.v, u.dout = (x.ctypes.data + base for x in (q, k, v, dout))
            u.in_stride = H * d
            u.len = b - a
            u.slope = float(slopes[h])
            st = ((si * H + h) * d * d) * f8
            u.s0 = (s0.ctypes.data + st) if s0 is not None else None
            u.ds = (ds.ctypes.data + st) if ds is not None else None
            ob = ((a * H + h) * d) * f8
            u.dq, u.dk, u.dv = (x.ctypes.data + ob for x in (dq, dk, dv))
            u.o_stride = H * d
            u.ds0 = ds0.ctypes.data + st
            idx += 1
    if _load().lto_backward(units, n * H, d, int(threads)) != 0:
        raise RuntimeError("lto_backward failed")
    return dq, dk, dv, ds0


def backward_batch(q, k, v, dout, slopes, s0=None, ds=None, threads=0):
    """backward_packed for [batch, L, H, d] inputs; returns [batch, L, H, d]
    gradients and [batch, H, d, d] ds0."""
    q = np.asarray(q)
    B, L, H, d = q.shape
    cu = np.arange(B + 1) * L
    flat = lambda x: np.asarray(x).reshape(B * L, H, d)
    dq, dk, dv, ds0 = backward_packed(flat(q), flat(k), flat(v), flat(dout), slopes, cu,
                                      s0=s0, ds=ds, threads=threads)
    return dq.reshape(B, L, H, d), dk.reshape(B, L, H, d), dv.reshape(B, L, H, d), ds0


def rope(x, positions, rope_dims, base):
    """Rotary position embedding on the first ``rope_dims`` features, rotate-half
    pairing: feature m and m + rope_dims/2 (m < rope_dims/2) rotate by the angle
    position * base^(-2m/rope_dims); features past rope_dims are unchanged.

    x: [..., T, H, d] (T = token axis -3); positions: [T] absolute positions.
    """
    x = np.asarray(x, np.float64)
    out = x.copy()
    if rope_dims == 0:
        return out
    half = rope_dims // 2
    m = np.arange(half, dtype=np.float64)
    theta = np.float64(base) ** (-2.0 * m / rope_dims)
    ang = np.asarray(positions, np.float64)[:, None] * theta[None, :]  # [T, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:rope_dims]
    out[..., :half] = x1 * c - x2 * s
    out[..., half:rope_dims] = x1 * s + x2 * c
    return out


def softmax_attention(q, k, v, rope_dims=64, base=10000.0, scale=None, pos0=0):
    """Causal softmax attention with grouped K/V heads and partial RoPE, fp64.

    q: [B, L, Hq, d]; k, v: [B, L, Hkv, d] with Hq a multiple of Hkv: query head
    h reads K/V head h // (Hq / Hkv). Token t sits at position pos0 + t.
    o_t = sum_{j <= t} softmax_j(scale * rope(q_t) . rope(k_j)) v_j, scale
    1/sqrt(d) by default. Returns o [B, L, Hq, d] fp64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    grp = Hq // Hkv
    sc = 1.0 / np.sqrt(d) if scale is None else np.float64(scale)
    pos = pos0 + np.arange(L)
    qr, kr = rope(q, pos, rope_dims, base), rope(k, pos, rope_dims, base)
    o = np.zeros((B, L, Hq, d))
    mask = np.tril(np.ones((L, L), bool))
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            s = sc * (qr[b, :, h] @ kr[b, :, g].T)
            s = np.where(mask, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            o[b, :, h] = p @ v[b, :, g]
    return o


def softmax_attention_rows(q, k, v, rows, rope_dims=64, base=10000.0, scale=None, pos0=0):
    """softmax_attention evaluated at the query rows ``rows`` only (for sequences
    too long for the full quadratic form): row t attends over keys 0..t.
    Returns [B, len(rows), Hq, d] fp64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    grp = Hq // Hkv
    sc = 1.0 / np.sqrt(d) if scale is None else np.float64(scale)
    rows = np.asarray(rows, np.int64)
    qr = rope(q[:, rows], pos0 + rows, rope_dims, base)
    kr = rope(k, pos0 + np.arange(L), rope_dims, base)
    o = np.zeros((B, len(rows), Hq, d))
    for b in range(B):
        for i, t in enumerate(rows):
            for h in range(Hq):
                g = h // grp
                s = sc * (kr[b, :t + 1, g] @ qr[b, i, h])
                p = np.exp(s - s.max())
                o[b, i, h] = (p / p.sum()) @ v[b, :t + 1, g]
    return o


def softmax_decode(q, k_new, v_new, k_cache, v_cache, lengths, rope_dims=64, base=10000.0,
                   scale=None):
    """One decode step over a KV cache, fp64.

    Sequence b's new token sits at position lengths[b]: rope(k_new) and v_new are
    appended at that position and rope(q) attends over positions 0..lengths[b].
    q: [B, Hq, d]; k_new, v_new: [B, Hkv, d]; k_cache, v_cache: [B, cap, Hkv, d]
    holding rope-applied keys and values at positions < lengths[b]. A length
    outside [0, cap) marks a padding row: zero output, cache untouched.
    Returns (o [B, Hq, d], k_cache, v_cache) with the new entries written.
    """
    q = np.asarray(q, np.float64)
    kc = np.array(k_cache, np.float64)
    vc = np.array(v_cache, np.float64)
    B, Hq, d = q.shape
    Hkv = kc.shape[2]
    grp = Hq // Hkv
    sc = 1.0 / np.sqrt(d) if scale is None else np.float64(scale)
    o = np.zeros((B, Hq, d))
    for b in range(B):
        n = int(lengths[b])
        if n < 0 or n >= kc.shape[1]:
            continue
        kc[b, n] = rope(np.asarray(k_new, np.float64)[b][None], [n], rope_dims, base)[0]
        vc[b, n] = np.asarray(v_new, np.float64)[b]
        qr = rope(q[b][None], [n], rope_dims, base)[0]
        for h in range(Hq):
            g = h // grp
            s = sc * (kc[b, :n + 1, g] @ qr[h])
            p = np.exp(s - s.max())
            o[b, h] = (p / p.sum()) @ vc[b, :n + 1, g]
    return o, kc, vc
