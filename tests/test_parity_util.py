"""CPU checks of the parity helpers the GPU tests use (no GPU needed).

The row bound exists because the per-head relative L2 error cannot see a few
wrong rows in a long sequence; these tests plant such rows in an otherwise
correct output and show that the per-head bound passes while the row bound
fails.
"""

import numpy as np
import pytest

from parity_util import (ROW_FACTOR, TOL_BF16, TOL_F32, boundary_row_err, boundary_rows,
                         max_rel_per_head, max_rel_states, parity_err, plan_segments, rel_l2,
                         slice_errors)


def _noisy(y, rel, seed):
    """y plus Gaussian noise of the given relative size per row (a stand-in for
    the bf16 rounding of a correct kernel)."""
    g = np.random.default_rng(seed)
    n = g.standard_normal(y.shape)
    n *= (np.linalg.norm(y, axis=-1, keepdims=True) / np.linalg.norm(n, axis=-1, keepdims=True)) * rel
    return y + n


def test_one_wrong_row_passes_head_bound_but_fails_row_bound():
    g = np.random.default_rng(1)
    L, d = 32768, 128
    y = g.standard_normal((L, d)) / np.sqrt(128)
    x = _noisy(y, 2e-3, 2)
    assert parity_err(x, y) <= TOL_BF16
    for bad in (0, 8191, 8192, 8193, 12345, L - 1):  # segment edges, an inner row, the last token
        xb = x.copy()
        xb[bad] = 0.0  # the row entirely wrong (e.g. a store that never happened)
        rel, row, idx = slice_errors(xb, y)
        assert rel <= TOL_BF16, rel  # the per-head bound alone would pass it
        assert idx == bad and row > 0.5
        assert parity_err(xb, y) > TOL_BF16


def test_one_wrong_column_of_one_row_fails_row_bound():
    g = np.random.default_rng(3)
    L, d = 4096, 128
    y = g.standard_normal((L, d)) / np.sqrt(128)
    x = _noisy(y, 2e-3, 4)
    x[777, 5] += 0.3  # one element off by ~3.4 typical element sizes
    assert rel_l2(x, y) <= TOL_BF16
    assert parity_err(x, y) > TOL_BF16


def test_small_early_rows_do_not_set_the_bound():
    """Rows with little history (norms far below the head's typical row norm)
    keep their absolute rounding error; the row bound is relative to the
    slice's RMS row norm, so they pass, and a wrong large row still fails."""
    g = np.random.default_rng(5)
    L, d = 2048, 128
    scale = np.minimum(1.0, (np.arange(L) + 1) / 512.0)[:, None]
    y = g.standard_normal((L, d)) * scale
    x = y + 2e-3 * g.standard_normal((L, d)) * np.sqrt(np.mean(np.sum(y * y, 1)) / d)
    assert parity_err(x, y) <= TOL_BF16
    x[1500] *= -1
    assert parity_err(x, y) > TOL_BF16


def test_fp32_bound_scales_with_the_tolerance():
    g = np.random.default_rng(6)
    y = g.standard_normal((1024, 128))
    x = _noisy(y, 1e-6, 7)
    assert parity_err(x, y) <= TOL_F32
    x[100] = _noisy(y[100:101], 1e-3, 8)[0]  # one row at 1e-3 relative
    assert rel_l2(x, y) <= TOL_F32 * 5
    assert parity_err(x, y) > TOL_F32


def test_non_finite_output_fails():
    y = np.ones((8, 128))
    x = y.copy()
    x[3, 3] = np.nan
    assert parity_err(x, y) == float("inf")


def test_packed_and_state_helpers_apply_the_row_bound():
    g = np.random.default_rng(9)
    cu = np.array([0, 3000, 3000, 9000])
    y = g.standard_normal((9000, 4, 128))
    x = _noisy(y, 1e-3, 10)
    assert max_rel_per_head(x, y, cu) <= TOL_BF16
    x[4321, 2] = 0.0
    assert max_rel_per_head(x, y, cu) > TOL_BF16
    s = g.standard_normal((2, 3, 128, 128))
    t = _noisy(s, 1e-3, 11)
    assert max_rel_states(t, s) <= TOL_BF16
    t[1, 2, 64] = 0.0  # one key row of one state
    assert max_rel_states(t, s) > TOL_BF16


def test_plan_rule_and_boundary_rows():
    """The documented launch plan of lt_prefill for the M1 layer (batch 1, 64
    heads, 32768 tokens: 4 segments of 8192) and the rows listed around its
    switches."""
    assert plan_segments(1, 32768, 64) == (4, 8192)
    assert plan_segments(1, 9000, 7) == (4, 2304)
    assert plan_segments(1, 4095, 64) == (1, 4095)
    assert plan_segments(4, 8192, 64) == (1, 8192)
    rows = boundary_rows(32768, 8192, 4, 2.0 ** (-1 / 8))
    for r in (0, 8190, 8191, 8192, 8193, 8194, 16384, 24576, 32767, 63, 64):
        assert r in rows
    # every sub-block edge (where warm-up ranges are cut) and its neighbours
    assert all(c in rows and c - 1 in rows for c in range(64, 32768, 64))
    # a wrong row at a listed boundary shows in the boundary error
    g = np.random.default_rng(12)
    y = g.standard_normal((32768, 128))
    x = y.copy()
    x[8192] = 0
    assert boundary_row_err(x, y, rows) > 1.0 / ROW_FACTOR / 2


@pytest.mark.parametrize("L", [1, 63, 64, 65])
def test_short_slices(L):
    g = np.random.default_rng(L)
    y = g.standard_normal((L, 128))
    assert parity_err(y, y) == 0.0
