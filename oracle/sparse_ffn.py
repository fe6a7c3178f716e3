"""Oracle for the sparse FFN token choice (test infrastructure only: used by
tests/ and nothing else; shares no code with the library).

RedKnot summary page, "Sparse FFN": only the top-k tokens by attention score
run the dense FFN; the rest keep their residual (identity). The score of a
token is its attention mass (oracle_mass_fp64). Reading taken for the ties
the pages leave open: equal scores go to the lower row, so the chosen set is
unique; zero, negative and NaN scores rank as zero.
"""

import numpy as np


def select_tokens(mass, cu_rows, keep, cu_keep=None):
    """Rows (ascending) of the keep[b] largest masses of each sequence; returns
    int32 [sum k_b] laid out by cu_keep (default: prefix sums of the clamped keep)."""
    mass = np.asarray(mass, dtype=np.float64)
    cu_rows = np.asarray(cu_rows, dtype=np.int64)
    keep = np.asarray(keep, dtype=np.int64)
    if cu_keep is None:
        k = np.minimum(keep, cu_rows[1:] - cu_rows[:-1])
        cu_keep = np.concatenate([[0], np.cumsum(np.maximum(k, 0))])
    cu_keep = np.asarray(cu_keep, dtype=np.int64)
    out = np.full(int(cu_keep[-1]), -1, dtype=np.int32)
    for b in range(len(keep)):
        r0, r1 = int(cu_rows[b]), int(cu_rows[b + 1])
        k = min(int(keep[b]), r1 - r0, int(cu_keep[b + 1] - cu_keep[b]))
        if k <= 0:
            continue
        score = mass[r0:r1].copy()
        score[~(score > 0)] = 0.0                      # NaN, zero and negative rank as zero
        rows = np.arange(r0, r1)
        order = np.lexsort((rows, -score))             # larger score first, then lower row
        out[cu_keep[b]:cu_keep[b] + k] = np.sort(rows[order[:k]])
    return out


def _bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _to_bf16_bits(x):
    """fp64 -> bf16 bits, rounded once to 8 significant bits, ties to even."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.ldexp(np.rint(m * 256.0), e - 8)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def silu(g):
    return g / (1.0 + np.exp(-g))


def swiglu_hidden(x_bits, rows, wg_bits, wu_bits):
    """h = bf16(silu(Wg x) * (Wu x)) for the chosen rows, in fp64 before the one rounding."""
    x = _bits_to_f64(np.asarray(x_bits)[np.asarray(rows)])
    g = x @ _bits_to_f64(wg_bits).T
    u = x @ _bits_to_f64(wu_bits).T
    return _to_bf16_bits(silu(g) * u)


def residual_down(x_bits, rows, h_bits, wd_bits):
    """The new bf16 rows x + Wd h (fp64, one rounding)."""
    x = _bits_to_f64(np.asarray(x_bits)[np.asarray(rows)])
    return _to_bf16_bits(x + _bits_to_f64(h_bits) @ _bits_to_f64(wd_bits).T)


def sparse_ffn(x_bits, rows, wg_bits, wu_bits, wd_bits):
    """Whole step on a host copy: returns (new x bits, h bits)."""
    h = swiglu_hidden(x_bits, rows, wg_bits, wu_bits)
    out = np.array(x_bits, copy=True)
    out[np.asarray(rows)] = residual_down(x_bits, rows, h, wd_bits)
    return out, h
