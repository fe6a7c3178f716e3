"""Pins for the oracle page-table builder (CPU only).

Every segment field is checked against what an explicit dense visibility
mask (brute force, built element by element) says: the page list must be
exactly the pages from the one holding the first key any query of the
segment can see through the page holding the last position, and the pair
count must be G times the number of true mask entries. On the full-size
workloads the totals are checked against closed forms:
  global query head, c cached and n new tokens: n*c + n(n+1)/2 pairs
  local query head with c = 0 and L >= W:       W(W+1)/2 + (L - W) W
  local query head with c + 1 >= W:             n W
"""

import numpy as np
import pytest

from oracle import bruteforce
from oracle.tables import TableError, build_tables
from workloads import ALL, LLAMA70B_32K, MISTRAL_8K, STACK64_128K, TINY, VARLEN_CHUNKED, realize
from tests.common import adhoc


def _check_against_mask(cached, new, classes, windows, page_of, hq, hkv, P, num_pages):
    t = build_tables(cached, new, classes, windows, page_of, hq, hkv, P, num_pages)
    G = hq // hkv
    s = 0
    row0 = 0
    pages_seen = 0
    klen_sum = 0
    for b in range(len(cached)):
        c, n = int(cached[b]), int(new[b])
        T = c + n
        for g in range(hkv):
            glob = bool(classes[g])
            M = bruteforce.visibility_mask(c, n, glob, int(windows[g]))
            cols = np.nonzero(M.any(axis=0))[0]
            j0 = int(cols.min())
            assert int(cols.max()) == T - 1
            first_lp, last_lp = j0 // P, (T - 1) // P
            assert t["k_pos0"][s] == first_lp * P
            assert t["k_len"][s] == T - first_lp * P
            assert t["q_row0"][s] == row0 and t["n_q"][s] == n and t["q_pos0"][s] == c
            assert t["kv_head"][s] == g and t["q_head0"][s] == g * G
            assert t["window"][s] == (0 if glob else windows[g])
            a, e = t["cu_pages"][s], t["cu_pages"][s + 1]
            assert a == pages_seen
            np.testing.assert_array_equal(t["page_list"][a:e], page_of[b, g, first_lp:last_lp + 1])
            pages_seen = e
            assert t["pairs"][s] == G * int(M.sum())
            assert t["cu_seqlens_k"][s] == klen_sum
            klen_sum += int(t["k_len"][s])
            s += 1
        row0 += n
    assert t["cu_seqlens_k"][s] == klen_sum
    assert len(t["page_list"]) == pages_seen
    np.testing.assert_array_equal(t["cu_seqlens_q"], np.concatenate([[0], np.cumsum(new)]))


SMALL = [
    (((0, 1),), 1), (((0, 17),), 16), (((5, 30),), 1), (((37, 100),), 17),
    (((0, 100), (37, 15), (5, 2)), 15), (((16, 16), (15, 1)), 16), (((100, 20),), 200),
    (((64, 64),), 50), (((0, 64),), 64), (((3, 13), (0, 50)), 2),
]


@pytest.mark.parametrize("seqs,W", SMALL)
@pytest.mark.parametrize("classes", [(1, 0), (0, 0), (0, 1, 1, 0)])
def test_segments_match_dense_mask(seqs, W, classes):
    hkv = len(classes)
    w = adhoc(hq=2 * hkv, hkv=hkv, d=8, page=16, window=W, classes=classes, seqs=seqs, seed=11)
    r = realize(w)
    _check_against_mask(r.cached_len, r.new_len, r.head_class[0], r.window[0], r.page_of[0],
                        w.hq, w.hkv, w.page, r.num_pages)


def _closed_form_pairs(c, n, W, glob):
    if glob:
        return n * c + n * (n + 1) // 2
    if c == 0 and n >= W:
        return W * (W + 1) // 2 + (n - W) * W
    if c + 1 >= W:
        return n * W
    return None


@pytest.mark.parametrize("w", ALL, ids=lambda w: w.name)
def test_workload_totals_match_closed_forms(w):
    r = realize(w)
    G = w.hq // w.hkv
    layers = range(w.layers) if w.layers <= 8 else [0, 7, 8, 9, 31, 63]
    for layer in layers:
        t = build_tables(r.cached_len, r.new_len, r.head_class[layer], r.window[layer], r.page_of[layer],
                         w.hq, w.hkv, w.page, r.num_pages)
        s = 0
        for b in range(r.num_seqs):
            c, n = int(r.cached_len[b]), int(r.new_len[b])
            T = c + n
            for g in range(w.hkv):
                glob = bool(r.head_class[layer, g])
                cf = _closed_form_pairs(c, n, w.window, glob)
                assert cf is not None
                assert t["pairs"][s] == G * cf
                lo = 0 if glob else max(0, c - w.window + 1)
                assert t["cu_pages"][s + 1] - t["cu_pages"][s] == (T - 1) // w.page - lo // w.page + 1
                s += 1


@pytest.mark.parametrize("W", [1, 5, 16, 17, 40])
@pytest.mark.parametrize("page", [1, 4, 16])
def test_retain_from_page_against_the_mask(W, page):
    """retain_lp: pages before it hold no key a later query can see; the page
    itself holds one (checked against the explicit mask of a longer sequence
    whose first c + n rows are this step)."""
    seqs = ((0, 1), (0, 23), (9, 7), (30, 2), (64, 64))
    w = adhoc(hq=4, hkv=2, d=8, page=page, window=W, classes=(1, 0), seqs=seqs)
    r = realize(w)
    t = build_tables(r.cached_len, r.new_len, r.head_class[0], r.window[0], r.page_of[0],
                     w.hq, w.hkv, w.page, r.num_pages)
    s = 0
    for b, (c, n) in enumerate(seqs):
        T = c + n
        for g in range(w.hkv):
            glob = bool(r.head_class[0, g])
            # rows T .. T + 2W + page of a continuation: the queries still to come
            future = bruteforce.visibility_mask(T, 2 * W + page + 1, glob, W)   # [rows][T + rows]
            seen = np.flatnonzero(future[:, :T].any(axis=0))
            first_needed = int(seen.min()) if seen.size else T
            lp = int(t["retain_lp"][s])
            assert lp * page <= first_needed
            assert first_needed < (lp + 1) * page or (glob and lp == 0)
            s += 1


def test_printed_pair_counts():
    """Pair totals of the three single-sequence workloads, from the closed forms
    written out by hand: global q-head L(L+1)/2, local W(W+1)/2 + (L-W)W."""
    expect = {
        TINY.name: 2 * 131_328 + 2 * 30_752,
        MISTRAL_8K.name: 4 * 33_558_528 + 28 * 7_864_832,
        LLAMA70B_32K.name: 8 * 536_887_296 + 56 * 65_012_736,
    }
    for w in (TINY, MISTRAL_8K, LLAMA70B_32K):
        r = realize(w)
        t = build_tables(r.cached_len, r.new_len, r.head_class[0], r.window[0], r.page_of[0],
                         w.hq, w.hkv, w.page, r.num_pages)
        assert int(t["pairs"].sum()) == expect[w.name]


def test_stack_class_draw_rules():
    r = realize(STACK64_128K)
    assert (r.head_class[:8] == 0).all()
    frac = r.head_class[8:].mean()
    assert 0.05 < frac < 0.25
    for w in (MISTRAL_8K, LLAMA70B_32K, VARLEN_CHUNKED):
        assert (realize(w).head_class.sum(axis=1) == 1).all()
    c = realize(VARLEN_CHUNKED).cached_len
    assert c.min() >= 2048 and c.max() <= 32768 and len(c) == 16


def test_errors():
    w = adhoc(hq=4, hkv=2, d=8, page=16, window=8, classes=(1, 0), seqs=((5, 40),))
    r = realize(w)
    args = (r.cached_len, r.new_len, r.head_class[0], r.window[0])
    po = r.page_of[0].copy()
    po[0, 1, 2] = -1                                   # inside the local head's visible range
    with pytest.raises(TableError) as e:
        build_tables(*args, po, 4, 2, 16, r.num_pages)
    assert e.value.kind == "range"
    po = r.page_of[0].copy()
    po[0, 0, 0] = r.num_pages                          # id past the pool
    with pytest.raises(TableError) as e:
        build_tables(*args, po, 4, 2, 16, r.num_pages)
    assert e.value.kind == "range"
    with pytest.raises(TableError) as e:
        build_tables(*args, r.page_of[0], 5, 2, 16, r.num_pages)
    assert e.value.kind == "invalid"
    with pytest.raises(TableError) as e:
        build_tables(r.cached_len, r.new_len, r.head_class[0], np.array([0, 0]), r.page_of[0], 4, 2, 16, r.num_pages)
    assert e.value.kind == "invalid"
    with pytest.raises(TableError) as e:
        build_tables(r.cached_len, np.array([0]), r.head_class[0], r.window[0], r.page_of[0], 4, 2, 16, r.num_pages)
    assert e.value.kind == "invalid"


def test_pages_before_the_window_may_be_absent():
    # a local head retains pages from floor(lo / P) on; earlier ids may be -1
    w = adhoc(hq=4, hkv=2, d=8, page=16, window=10, classes=(1, 0), seqs=((70, 20),))
    r = realize(w)
    po = r.page_of[0].copy()
    po[0, 1, :3] = -1                                  # lo = 61 -> first retained logical page 3
    t = build_tables(r.cached_len, r.new_len, r.head_class[0], r.window[0], po, 4, 2, 16, r.num_pages)
    assert t["k_pos0"][1] == 48
