"""Oracle page-table builder (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module. It shares no code with the library under test.

What it computes, one layer at a time (RedKnot summary page, sections
"Head-Class Sparsification" and "SegPaged Attention"): the KV cache is stored
as pages segmented per (layer, KV head); a global head keeps its sequence's
full causal context, a local head keeps only a sliding window; each head
physically stores only the pages it needs. The block table is the
logical-to-physical page map of the KV-cache management page (section 3.1).

Readings taken where the pages are silent:
  * a local window of W holds the W most recent keys including the query
    itself: key j is visible to query i iff i - W < j <= i;
  * GQA is contiguous: query head h reads KV head h // G, G = hq / hkv;
  * the class is per (layer, KV head) and shared by its G query heads;
  * segment order within a layer is s = b * hkv + g; window 0 marks a
    global segment;
  * a local segment's page list starts at the page that holds the first key
    visible to its first query, lo = max(0, c_b - W + 1), so its first
    position is k_pos0 = floor(lo / P) * P; it runs to the page holding the
    last position T_b - 1; k_len = T_b - k_pos0 counts from that aligned
    start.

Parity pins: tests/test_oracle_tables.py checks every field against sets
derived from an explicit dense visibility mask (brute force) and against
closed forms for the counts.
"""

import numpy as np


class TableError(ValueError):
    """Raised for inputs the definition does not cover; .kind is 'invalid' or 'range'."""

    def __init__(self, kind, msg):
        super().__init__(msg)
        self.kind = kind


def build_tables(cached_len, new_len, head_class, window, page_of, hq, hkv, page, num_pages):
    """Build one layer's segment tables.

    cached_len, new_len : int [S]            c_b >= 0, n_b >= 1
    head_class          : int [hkv]          1 global, 0 local
    window              : int [hkv]          W >= 1 for local heads (ignored for global)
    page_of             : int [S][hkv][max_lp] physical page id per logical page, -1 none
    Returns a dict of numpy arrays (int32, pairs int64).
    """
    cached_len = np.asarray(cached_len, dtype=np.int64)
    new_len = np.asarray(new_len, dtype=np.int64)
    head_class = np.asarray(head_class)
    window = np.asarray(window, dtype=np.int64)
    page_of = np.asarray(page_of)
    if hkv <= 0 or hq <= 0 or hq % hkv != 0:
        raise TableError("invalid", "query heads must be a positive multiple of KV heads")
    if page <= 0:
        raise TableError("invalid", "page size must be positive")
    G = hq // hkv
    nseq = cached_len.shape[0]
    max_lp = page_of.shape[2]

    cu_q = [0]
    q_row0, n_q, q_pos0, kv_head, q_head0 = [], [], [], [], []
    win_out, k_pos0, k_len = [], [], []
    cu_k, cu_pages, page_list, pairs, retain = [0], [0], [], [], []

    for b in range(nseq):
        c = int(cached_len[b])
        n = int(new_len[b])
        if c < 0 or n < 1:
            raise TableError("invalid", f"sequence {b}: need c >= 0 and n >= 1")
        T = c + n
        for g in range(hkv):
            is_global = int(head_class[g]) != 0
            if is_global:
                W = 0
                first_pos = 0
            else:
                W = int(window[g])
                if W < 1:
                    raise TableError("invalid", f"kv head {g}: local window must be >= 1")
                first_pos = (max(0, c - W + 1) // page) * page
            first_lp = first_pos // page
            last_lp = (T - 1) // page
            if last_lp >= max_lp:
                raise TableError("range", f"sequence {b} needs logical page {last_lp} >= max_lp")
            for lp in range(first_lp, last_lp + 1):
                pid = int(page_of[b, g, lp])
                if pid < 0 or pid >= num_pages:
                    raise TableError("range", f"segment ({b},{g}) logical page {lp}: bad id {pid}")
                page_list.append(pid)

            # visible keys of query i = c + t: |{j : lo(i) <= j <= i}|
            i = c + np.arange(n, dtype=np.int64)
            if is_global:
                count = i + 1
            else:
                count = np.minimum(i + 1, W)

            q_row0.append(cu_q[-1])
            n_q.append(n)
            q_pos0.append(c)
            kv_head.append(g)
            q_head0.append(g * G)
            win_out.append(W)
            k_pos0.append(first_pos)
            k_len.append(T - first_pos)
            cu_k.append(cu_k[-1] + T - first_pos)
            cu_pages.append(len(page_list))
            pairs.append(G * int(count.sum()))
            # pages a later query (position >= T) can still see: a local head's
            # next query starts its window at T - W + 1, a global head sees all
            retain.append(0 if is_global else max(0, T - W + 1) // page)
        cu_q.append(cu_q[-1] + n)

    i32 = lambda x: np.asarray(x, dtype=np.int32)  # noqa: E731
    return {
        "q_row0": i32(q_row0), "n_q": i32(n_q), "q_pos0": i32(q_pos0),
        "kv_head": i32(kv_head), "q_head0": i32(q_head0), "window": i32(win_out),
        "k_pos0": i32(k_pos0), "k_len": i32(k_len),
        "cu_seqlens_q": i32(cu_q), "cu_seqlens_k": i32(cu_k), "cu_pages": i32(cu_pages),
        "page_list": i32(page_list), "pairs": np.asarray(pairs, dtype=np.int64),
        "retain_lp": i32(retain),
        "G": G, "page": page, "hq": hq, "hkv": hkv,
    }
