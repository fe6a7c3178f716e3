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
