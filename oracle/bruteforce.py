"""Brute-force dense attention with an explicit boolean mask (test infrastructure only).

Only tests/ may import this module. It is the pin for the paged oracle on
tiny inputs: it never sees a page, a page table or a visible-range formula.
It takes each sequence's dense logical K/V (before any paging), builds the
full [n x T] visibility mask element by element from the definition, and
applies a textbook softmax, all in float64 NumPy.

Visibility (RedKnot summary page, "Head-Class Sparsification": global heads
see the whole context, local heads a sliding window; the window reading is
"the W most recent keys, the query's own key included"):
    M[i, j] = (j <= i) and (global or i - j < W)
"""

import numpy as np


def visibility_mask(c, n, is_global, W):
    """Boolean [n][c+n]: row t is the query at absolute position c + t."""
    T = c + n
    M = np.zeros((n, T), dtype=bool)
    for t in range(n):
        i = c + t
        for j in range(T):
            M[t, j] = (j <= i) and (is_global or (i - j) < W)
    return M


def dense_masked_attention(q, k, v, c, is_global, W, scale):
    """q [n][D], k/v [c+n][D] (float64). Returns (O [n][D], lse [n])."""
    n = q.shape[0]
    M = visibility_mask(c, n, is_global, W)
    S = (q @ k.T) * scale
    S = np.where(M, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    denom = E.sum(axis=1, keepdims=True)
    O = (E / denom) @ v
    return O, (m + np.log(denom))[:, 0]


def layer_reference(q, k_seq, v_seq, cached_len, new_len, head_class, window, hq, hkv, scale):
    """All queries of a layer, dense. q [sum n][hq][D] float64; k_seq/v_seq:
    list over sequences of [c_b+n_b][hkv][D] float64 (dense logical rows).
    Returns O [sum n][hq][D], lse [sum n][hq]."""
    G = hq // hkv
    D = q.shape[-1]
    O = np.zeros((q.shape[0], hq, D))
    L = np.zeros((q.shape[0], hq))
    row = 0
    for b in range(len(cached_len)):
        c, n = int(cached_len[b]), int(new_len[b])
        for h in range(hq):
            g = h // G
            o, lse = dense_masked_attention(q[row:row + n, h, :], k_seq[b][:, g, :], v_seq[b][:, g, :],
                                            c, bool(head_class[g]), int(window[g]), scale)
            O[row:row + n, h, :] = o
            L[row:row + n, h] = lse
        row += n
    return O, L
