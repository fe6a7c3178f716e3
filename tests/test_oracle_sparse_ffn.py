"""Pins of the sparse FFN token choice (oracle/sparse_ffn.py) against the
properties that define it: exactly k rows per sequence, ascending, every
chosen score >= every unchosen one, ties at the boundary to the lower rows,
and the clamps (k > n, output room)."""

import numpy as np
import pytest

from oracle.sparse_ffn import select_tokens


def _check(mass, cu, keep, out):
    off = 0
    for b in range(len(keep)):
        r0, r1 = cu[b], cu[b + 1]
        k = min(keep[b], r1 - r0)
        sel = out[off:off + k]
        off += k
        assert len(sel) == k and np.all(np.diff(sel) > 0) and np.all((sel >= r0) & (sel < r1))
        s = np.where(mass[r0:r1] > 0, mass[r0:r1], 0.0)
        chosen = np.zeros(r1 - r0, bool)
        chosen[sel - r0] = True
        if 0 < k < r1 - r0:
            lo, hi = s[chosen].min(), s[~chosen].max()
            assert lo >= hi
            # at equal scores a chosen row never comes after an unchosen one
            tie_rows_in = np.flatnonzero(chosen & (s == lo))
            tie_rows_out = np.flatnonzero(~chosen & (s == lo))
            if lo == hi and tie_rows_in.size and tie_rows_out.size:
                assert tie_rows_in.max() < tie_rows_out.min()


@pytest.mark.parametrize("seed", range(6))
def test_selection_properties(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    n = rng.integers(1, 60, size=5)
    cu = np.concatenate([[0], np.cumsum(n)])
    mass = np.round(rng.random(cu[-1]) * 4) / 4           # many ties
    mass[rng.random(cu[-1]) < 0.1] = 0.0
    keep = np.array([rng.integers(0, x + 3) for x in n])
    out = select_tokens(mass, cu, keep)
    _check(mass, cu, keep, out)


def test_selection_small_by_hand():
    mass = np.array([0.5, 2.0, 0.5, 1.0, np.nan, -1.0, 0.5])
    assert select_tokens(mass, [0, 7], [3]).tolist() == [0, 1, 3]       # 2.0, 1.0, then the first 0.5
    assert select_tokens(mass, [0, 7], [5]).tolist() == [0, 1, 2, 3, 6]
    assert select_tokens(mass, [0, 7], [7]).tolist() == list(range(7))  # NaN and -1 rank as zero, last
    assert select_tokens(mass, [0, 3, 7], [1, 2]).tolist() == [1, 3, 6]  # second sequence: 1.0 and the first 0.5
    assert select_tokens(mass, [0, 3, 7], [5, 0], cu_keep=[0, 2, 2]).tolist() == [0, 1]   # room clamps


def _bits(x):
    from oracle.sparse_ffn import _to_bf16_bits
    return _to_bf16_bits(np.asarray(x, dtype=np.float64))


def test_ffn_by_hand():
    """d_model 2, d_ff 2, one chosen row: the SwiGLU block written out."""
    import math
    from oracle.sparse_ffn import sparse_ffn, _bits_to_f64
    x = np.array([[1.0, 0.5], [2.0, -1.0]])
    wg = np.array([[1.0, 0.0], [0.5, 1.0]])
    wu = np.array([[2.0, 1.0], [0.0, -1.0]])
    wd = np.array([[1.0, 0.25], [-0.5, 1.0]])
    out, h = sparse_ffn(_bits(x), [1], _bits(wg), _bits(wu), _bits(wd))
    g = [2.0, 0.0]                                     # Wg x1 = (2, 1 - 1)
    u = [3.0, 1.0]                                     # Wu x1 = (4 - 1, 1)
    hv = [g[0] / (1 + math.exp(-g[0])) * u[0], 0.0]
    assert np.array_equal(h[0], _bits(hv))
    hb = _bits_to_f64(_bits(hv))
    y = [2.0 + 1.0 * hb[0] + 0.25 * hb[1], -1.0 - 0.5 * hb[0] + 1.0 * hb[1]]
    assert np.array_equal(out[1], _bits(y))
    assert np.array_equal(out[0], _bits(x[0]))        # not chosen: the residual identity


def test_ffn_closed_forms():
    from oracle.sparse_ffn import sparse_ffn, silu, _bits_to_f64
    rng = np.random.Generator(np.random.PCG64(3))
    x = _bits(rng.standard_normal((9, 8)))
    wg, wd = _bits(rng.standard_normal((16, 8))), _bits(rng.standard_normal((8, 16)))
    out, h = sparse_ffn(x, [2, 5], wg, _bits(np.zeros((16, 8))), wd)    # zero up projection: no change
    assert np.array_equal(out, x) and not _bits_to_f64(h).any()        # (signed zeros)
    g = np.linspace(-6, 6, 25)
    np.testing.assert_allclose(silu(g) - silu(-g), g, atol=1e-12)      # silu(g) - silu(-g) = g
    assert silu(0.0) == 0.0
