"""The library's host table builder (segkv_build_head_tables) against the
oracle's, bit for bit, on every workload (every layer of the 64-layer stack)
and on small ragged cases; plus the work list's coverage and order."""

import numpy as np
import pytest

import head_segmented_paged_amd as H
from oracle.tables import build_tables
from tests.common import adhoc
from workloads import ALL, STACK64_128K, realize

FIELDS = ("q_row0", "n_q", "q_pos0", "kv_head", "window", "k_pos0", "k_len",
          "cu_seqlens_q", "cu_seqlens_k", "cu_pages", "page_list", "pairs", "retain_lp")


class FakeDev:
    def __init__(self, p):
        self.p = p

    def data_ptr(self):
        return self.p


def _ctx(w, num_pages):
    return H.segkv_create(FakeDev(1 << 20), FakeDev(1 << 21), w.hq, w.hkv, w.d, w.page, num_pages=num_pages)


def _compare(w, r, layer, ctx):
    lib = H.segkv_build_head_tables(ctx, r.cached_len, r.new_len, r.head_class[layer], r.window[layer],
                                    r.page_of[layer])
    ora = build_tables(r.cached_len, r.new_len, r.head_class[layer], r.window[layer], r.page_of[layer],
                       w.hq, w.hkv, w.page, r.num_pages)
    for f in FIELDS:
        a, b = lib[f], ora[f]
        assert a.dtype == b.dtype, f
        np.testing.assert_array_equal(a, b, err_msg=f)
    np.testing.assert_array_equal(lib["page_off"], ora["cu_pages"][:-1])
    assert lib["total_pairs"] == int(ora["pairs"].sum())
    return lib


def _waves(w, lib):
    """Wavefronts per prefill workgroup: eight for pages of at least one tile
    when the layer's mean visible keys per query row and KV head reach 1024
    for head dim 128, 2048 otherwise (sum of visible pairs over its segments,
    from the oracle-checked total_pairs, against the cut x rows), four
    otherwise."""
    G = w.hq // w.hkv
    cut = 1024 if w.d == 128 else 2048
    long_context = lib["total_pairs"] >= cut * G * w.hkv * lib["total_q_rows"]
    return 8 if w.page >= 64 and long_context else 4


def _window(waves, decode):
    """Cohort window of the work list: 8 XCDs x the workgroups one XCD holds
    (32 CUs x 8 waves / waves per workgroup; decode lists use 64)."""
    return 8 * (64 if decode else 32 * 8 // waves)


def _check_order(work, WINDOW):
    """Longest first between windows; inside a window, each XCD's share
    (positions x, x+8, ...) in descending (segment, row, head) order, and the
    shares one after another in ascending order."""
    tiles = work[:, 3]
    for a in range(0, len(work), WINDOW):
        win = work[a:a + WINDOW]
        if a + WINDOW < len(work):
            assert tiles[a:a + WINDOW].min() >= tiles[a + WINDOW:].max()
        for x in range(8):
            share = [tuple(int(v) for v in u[[0, 1, 2, 4]]) for u in win[x::8]]
            assert all(a > b for a, b in zip(share, share[1:]))
        # the XCDs' shares follow one another in (segment, row, head) order,
        # XCD 0 first in even windows and XCD 7 first in odd ones
        order = range(min(8, len(win)))
        if (a // WINDOW) % 2 == 1:
            order = [x for x in reversed(range(8)) if x < len(win)]
        lows = [tuple(win[x::8][-1][[0, 1, 2, 4]]) for x in order]
        highs = [tuple(win[x::8][0][[0, 1, 2, 4]]) for x in order]
        for i in range(len(lows) - 1):
            assert highs[i] < lows[i + 1]


def _check_work(lib, w):
    G = w.hq // w.hkv
    work = lib["work"]
    rows, heads = lib["unit_rows"], lib["unit_heads"]
    decode = w.page >= 64 and G <= 32 and int(lib["n_q"].max()) <= 32 // G
    waves = _waves(w, lib)
    prefill_heads = max(h for h in (1, 2, 4, 8) if h <= waves and G % h == 0)
    assert (heads, rows) == ((G, 32 // G) if decode else (prefill_heads, 32 * waves // prefill_heads))
    # fields 6..9: the page ids of the unit's first four tiles, read from the
    # (oracle-checked) page list; -1 past the unit's run or the segment's pages
    seg, t0, nt = work[:, 0].astype(np.int64), work[:, 4].astype(np.int64), work[:, 3].astype(np.int64)
    off, n_pages = lib["cu_pages"][seg], lib["cu_pages"][seg + 1] - lib["cu_pages"][seg]
    for i in range(4):
        lp = (t0 + i) * 64 // w.page
        ok = (i < nt) & (lp < n_pages)
        want = np.where(ok, lib["page_list"][np.where(ok, off + lp, 0)], -1)
        np.testing.assert_array_equal(work[:, 6 + i], want, err_msg=f"page of tile {i}")
    assert (work[:, 10:] == 0).all()
    _check_order(work, _window(waves, decode))
    # blocks: every (segment, head, row) in exactly one block; a block's units
    # cut its natural run of tiles into consecutive pieces
    blocks = {}
    for u in work:
        blocks.setdefault((int(u[0]), int(u[1]), int(u[2])), []).append(u)
    for s in range(lib["num_segments"]):
        n = lib["n_q"][s]
        g = lib["kv_head"][s]
        cnt = np.zeros((G, n), np.int32)
        for (seg, r0, h0) in [b for b in blocks if b[0] == s]:
            assert g * G <= h0 and h0 + heads <= (g + 1) * G and r0 % rows == 0
            cnt[h0 - g * G: h0 - g * G + heads, r0: min(r0 + rows, n)] += 1
        assert (cnt == 1).all()
    merges = {(int(m[0]), int(m[1]), int(m[2])): m for m in lib["merge"]}
    assert len(merges) == lib["num_merges"] == len(lib["merge"])
    for m in lib["merge"]:   # output rows of the block, straight from its segment
        seg, r0 = int(m[0]), int(m[1])
        assert m[5] == lib["q_row0"][seg] + r0 and m[6] == min(rows, lib["n_q"][seg] - r0) and m[7] == 0
    seen_parts = []
    for key, units in blocks.items():
        seg, r0, h0 = key
        c, W, k0 = lib["q_pos0"][seg], lib["window"][seg], lib["k_pos0"][seg]
        last = c + min(r0 + rows, lib["n_q"][seg]) - 1
        lo = 0 if W == 0 else max(0, c + r0 - W + 1)
        t0, t1 = (lo - k0) // 64, -(-(last + 1 - k0) // 64)
        runs = sorted((int(u[4]), int(u[3]), int(u[5])) for u in units)
        assert runs[0][0] == t0 and runs[-1][0] + runs[-1][1] == t1
        for (a, na, _), (b, _, _) in zip(runs, runs[1:]):
            assert a + na == b and na >= 1
        if len(runs) == 1:
            assert runs[0][2] == -1 and key not in merges
        else:
            m = merges[key]
            parts = sorted(r[2] for r in runs)
            assert parts == list(range(m[3], m[3] + m[4]))
            seen_parts += parts
    assert sorted(seen_parts) == list(range(lib["num_parts"]))
    # partial results, then (units of 256 pairs) the persistent kernel's work queues
    queue = 256 if rows * heads == 256 else 0
    assert lib["workspace_bytes"] == lib["num_parts"] * 4 * rows * heads * (w.d + 2) + queue


@pytest.mark.parametrize("w", [x for x in ALL if x.layers == 1], ids=lambda w: w.name)
def test_single_layer_workloads(w):
    r = realize(w)
    ctx = _ctx(w, r.num_pages)
    lib = _compare(w, r, 0, ctx)
    _check_work(lib, w)


def test_stack_all_layers():
    w = STACK64_128K
    r = realize(w)
    ctx = _ctx(w, r.num_pages)
    for layer in range(w.layers):
        lib = _compare(w, r, layer, ctx)
        if layer in (0, 8, 63):
            work = lib["work"]
            _check_order(work, _window(_waves(w, lib), False))
            assert len(work) == 8 * (131072 // lib["unit_rows"])


SMALL = [((0, 1),), ((0, 17),), ((5, 30),), ((37, 100),), ((0, 100), (37, 15), (5, 2)),
         ((16, 16), (15, 1)), ((100, 20),), ((64, 64),), ((3, 13), (0, 50), (200, 33))]


@pytest.mark.parametrize("max_run", [1, 2, 3, 7])
@pytest.mark.parametrize("seqs", [((0, 300),), ((100, 20),), ((0, 100), (37, 15), (5, 2)), ((200, 130), (3, 13))])
@pytest.mark.parametrize("page", [16, 64])
def test_forced_splits(max_run, seqs, page):
    w = adhoc(hq=8, hkv=2, d=64, page=page, window=70, classes=(1, 0), seqs=seqs, seed=max_run + page)
    r = realize(w)
    ctx = _ctx(w, r.num_pages)
    lib = H.segkv_build_head_tables(ctx, r.cached_len, r.new_len, r.head_class[0], r.window[0], r.page_of[0],
                                    max_unit_tiles=max_run)
    lib.update({k: lib["seg_desc"][:, i] for i, k in enumerate(("q_row0", "n_q", "q_pos0", "kv_head", "window",
                                                                "k_pos0", "k_len", "page_off"))})
    _check_work(lib, w)
    if page < 64:
        assert lib["num_parts"] == 0          # the small-page kernel has no split path
    else:
        never = H.segkv_build_head_tables(ctx, r.cached_len, r.new_len, r.head_class[0], r.window[0],
                                          r.page_of[0], max_unit_tiles=-1)
        assert (lib["work"][:, 3] <= max_run).all()
        assert (lib["num_parts"] > 0) == (never["work"][:, 3].max() > max_run)


def test_automatic_split_policy():
    """Splits exactly where list scheduling cannot balance: the 8K layer's longest
    block (128 tiles) exceeds 3/4 of the mean load per workgroup slot."""
    by = {x.name: x for x in ALL}
    for name, expect in (("mistral7b_like_l8192", True), ("llama70b_like_l32768", False),
                         ("varlen16_chunk2048", False), ("tiny_gqa2_l512", False), ("decode32_l32768", True)):
        w = by[name]
        r = realize(w)
        ctx = _ctx(w, r.num_pages)
        lib = H.segkv_build_head_tables(ctx, r.cached_len, r.new_len, r.head_class[0], r.window[0],
                                        r.page_of[0])
        assert (lib["num_parts"] > 0) == expect, name
        if expect and lib["unit_rows"] * lib["unit_heads"] == 128:
            total = int(lib["work"][:, 3].sum())
            assert lib["work"][:, 3].max() <= max(16, -(-total // 1024)) + 1
        if expect and lib["unit_rows"] * lib["unit_heads"] == 256:   # two-block kernel: a slot's mean load
            total = int(lib["work"][:, 3].sum())
            assert -(-total // 512) < lib["work"][:, 3].max() <= max(16, -(-total // 256)) + 1
        if expect and lib["unit_rows"] * lib["unit_heads"] < 128:      # decode: about one unit per wave slot
            assert len(lib["work"]) >= 8 * 256 * 0.9
        never = H.segkv_build_head_tables(ctx, r.cached_len, r.new_len, r.head_class[0], r.window[0],
                                          r.page_of[0], max_unit_tiles=-1)
        assert never["num_parts"] == 0


@pytest.mark.parametrize("seqs", SMALL)
@pytest.mark.parametrize("W", [1, 16, 17, 64])
@pytest.mark.parametrize("shape", [(4, 2, (1, 0)), (8, 2, (0, 1)), (3, 3, (0, 1, 1)), (8, 1, (0,))])
@pytest.mark.parametrize("page", [16, 64])
def test_small_cases(seqs, W, shape, page):
    hq, hkv, classes = shape
    w = adhoc(hq=hq, hkv=hkv, d=64, page=page, window=W, classes=classes, seqs=seqs, seed=W + page)
    r = realize(w)
    ctx = _ctx(w, r.num_pages)
    lib = _compare(w, r, 0, ctx)
    _check_work(lib, w)
