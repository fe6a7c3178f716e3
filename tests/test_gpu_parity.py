"""GPU parity: the HIP path (paged write, host tables, fused attention, all
through the C ABI) against the fp64 oracle on the same seeded inputs.

Bar (fp32 output, bf16 inputs, fp32 accumulation): max-abs <= 1e-2 and
mean-abs <= 1e-3 against the oracle, LSE within 2e-3. The bf16 output mode
must equal the fp32 output rounded to nearest-even, bit for bit. Page
tables are bit-exact (tests/test_tables_vs_oracle.py); the paged write is
bit-exact against the oracle's own scatter. Outputs are bitwise invariant
under physical page relabelling, reruns and NaN-poisoned free slots.

Small cases, the 8K layer and the chunked varlen batch run every query; the
32K layer and the 128K stack (two layers of each class) run sampled rows
(first and last rows, window-edge and page-boundary rows, 256 seeded-uniform
rows per head), which the oracle computes one by one.
"""

import os

import numpy as np
import pytest
import torch

from oracle import paged as opaged
from oracle import tables as otables
from tests.common import adhoc
from tests.gpu_helpers import GpuLayer, compare, device_pools, host_bits, sample_rows, say
from workloads import (DECODE_32K, LLAMA70B_32K, MISTRAL_8K, STACK64_128K, TINY, VARLEN_CHUNKED, layer_tensors,
                       realize)
from workloads.gen import relabel_pages

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def oracle_queries(w, r, layer, bits, queries, page_of=None):
    """Oracle results for (b, h, t) queries of one layer: own tables, own paged write."""
    po = r.page_of[layer] if page_of is None else page_of
    tab = otables.build_tables(r.cached_len, r.new_len, r.head_class[layer], r.window[layer], po,
                               w.hq, w.hkv, w.page, r.num_pages)
    kp, vp = opaged.empty_pools(r.num_pages, w.page, w.d)
    opaged.scatter_pages(kp, vp, po, r.cached_len, r.new_len, bits["k_cached"], bits["v_cached"],
                         bits["k_new"], bits["v_new"])
    o, lse = opaged.attention(kp, vp, bits["q"], tab, queries)
    del kp, vp
    return o, lse, tab


def all_queries(w, r):
    out = []
    for b in range(r.num_seqs):
        n = int(r.new_len[b])
        for h in range(w.hq):
            out.append(np.stack([np.full(n, b), np.full(n, h), np.arange(n)], 1))
    return np.concatenate(out).astype(np.int32)


def sampled_queries(w, r, layer, seed, n_uniform=256, heads=None):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for b in range(r.num_seqs):
        c, n = int(r.cached_len[b]), int(r.new_len[b])
        for h in (range(w.hq) if heads is None else heads):
            g = h // (w.hq // w.hkv)
            W = int(r.window[layer][g]) or w.window
            t = sample_rows(n, c, W, w.page, rng, n_uniform=n_uniform)
            out.append(np.stack([np.full(len(t), b), np.full(len(t), h), t], 1))
    return np.concatenate(out).astype(np.int32)


def run_case(w, layer=0, queries="all", seed=0, o_dtype=torch.float32, **kw):
    r = realize(w)
    say(f"[case] {w.name} layer {layer} hq {w.hq} hkv {w.hkv} D {w.d} P {w.page} "
        f"seqs {list(zip(r.cached_len.tolist(), r.new_len.tolist()))[:4]}")
    t = layer_tensors(w, r, layer, device="cuda")
    gl = GpuLayer(w, r, layer, t, **kw)
    o, lse = gl.run(o_dtype)
    bits = {k: host_bits(v) for k, v in t.items()}
    q = all_queries(w, r) if queries == "all" else sampled_queries(w, r, layer, seed)
    oo, ol, tab = oracle_queries(w, r, layer, bits, q, page_of=kw.get("page_of"))
    stats = compare(o, lse, oo, ol, q, tab, w.hkv)
    say(f"[ok] {w.name} layer {layer}: {stats}")
    return o, lse, gl


def test_tiny_all_rows():
    o, lse, gl = run_case(TINY)
    # bf16 output is the fp32 output rounded to nearest even
    ob, _ = gl.attention(torch.bfloat16, with_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(ob, o.to(torch.bfloat16))


RAGGED = [
    # (hq, hkv, d, page, window, classes, seqs)
    (4, 2, 64, 16, 64, (1, 0), ((0, 333),)),
    (8, 2, 128, 64, 100, (0, 1), ((0, 200), (37, 301), (1000, 77))),
    (4, 4, 128, 16, 17, (0, 1, 0, 1), ((5, 130), (64, 64))),
    (8, 1, 128, 32, 1, (0,), ((0, 97),)),
    (16, 2, 64, 128, 300, (0, 0), ((250, 260), (0, 1))),
    (6, 3, 128, 256, 40, (1, 0, 0), ((700, 45), (3, 250))),
    (2, 2, 64, 64, 2000, (0, 1), ((0, 513),)),
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: f"hq{c[0]}_kv{c[1]}_d{c[2]}_p{c[3]}_w{c[4]}")
def test_ragged_all_rows(case):
    hq, hkv, d, page, window, classes, seqs = case
    run_case(adhoc(hq=hq, hkv=hkv, d=d, page=page, window=window, classes=classes, seqs=seqs, seed=hq * d + page))


SPLIT = [
    # (hq, hkv, d, page, window, classes, seqs, longest run in tiles)
    (8, 2, 128, 64, 100, (0, 1), ((0, 200), (37, 301), (1000, 77)), 1),
    (16, 2, 64, 128, 300, (0, 0), ((250, 260), (0, 1)), 2),
    (6, 3, 128, 256, 40, (1, 0, 0), ((700, 45), (3, 250)), 3),
    (4, 4, 64, 64, 1, (1, 1, 0, 0), ((0, 400), (130, 7)), 2),
    (4, 1, 128, 64, 500, (1,), ((900, 160),), 5),
]


@pytest.mark.parametrize("case", SPLIT, ids=lambda c: f"hq{c[0]}_kv{c[1]}_d{c[2]}_p{c[3]}_run{c[7]}")
def test_split_kv_all_rows(case):
    """Blocks cut into short runs: partial results through the workspace and the
    merge pass, every row against the oracle; bf16 output is RNE of fp32."""
    hq, hkv, d, page, window, classes, seqs, run = case
    w = adhoc(hq=hq, hkv=hkv, d=d, page=page, window=window, classes=classes, seqs=seqs, seed=hq * d + run)
    o, lse, gl = run_case(w, max_unit_tiles=run)
    assert gl.host["num_parts"] > 0 and gl.host["num_merges"] > 0
    ob, _ = gl.attention(torch.bfloat16, with_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(ob, o.to(torch.bfloat16))


WIDE = [
    # long contexts (mean visible keys per row >= 2048): eight-wave units of 256
    # (row, head) pairs; (hq, hkv, d, page, window, classes, seqs, run: 0 automatic)
    (8, 1, 128, 64, 0, (1,), ((3000, 300),), 0),
    (8, 1, 128, 64, 0, (1,), ((3000, 300),), 4),
    (4, 2, 64, 128, 3000, (1, 0), ((2500, 200), (4000, 77)), 0),
    (2, 2, 128, 256, 0, (1, 1), ((2100, 513),), 3),
    (16, 2, 128, 64, 2500, (0, 1), ((5000, 100), (2200, 33)), 0),
    # G = 4 and G = 2 at head dim 128: the two-block kernel with 4 x 64 and
    # 2 x 128 units (G = 4 is the 128K stack's shape)
    (8, 2, 128, 64, 1500, (1, 0), ((2500, 333),), 0),
    (8, 2, 128, 64, 2200, (0, 1), ((3000, 200), (2100, 65)), 5),
    (4, 2, 128, 64, 0, (1, 1), ((2049, 130),), 0),
    (4, 1, 128, 128, 2100, (0,), ((2500, 700),), 0),
]


@pytest.mark.parametrize("case", WIDE, ids=lambda c: f"hq{c[0]}_kv{c[1]}_d{c[2]}_p{c[3]}_run{c[7]}")
def test_wide_units_all_rows(case):
    """Eight-wave units (one K/V stream for 256 pairs), with and without split
    runs, G from 1 to 8: every row against the oracle; bf16 output is RNE of
    fp32."""
    hq, hkv, d, page, window, classes, seqs, run = case
    w = adhoc(hq=hq, hkv=hkv, d=d, page=page, window=window, classes=classes, seqs=seqs, seed=hq * 7 + d + run)
    o, lse, gl = run_case(w, max_unit_tiles=run if run else -1)
    assert gl.host["unit_rows"] * gl.host["unit_heads"] == 256
    assert (gl.host["num_parts"] > 0) == (run > 0)
    ob, _ = gl.attention(torch.bfloat16, with_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(ob, o.to(torch.bfloat16))


PERSISTENT = [
    # (hq, hkv, classes, seqs, longest run in tiles: -1 none); G = 4 with 510
    # units, or 258: two past the CU count, so nearly every workgroup finds
    # its queue empty at once; G = 1 (256 rows x 1 head) and G = 8 (32 rows x
    # 8 heads) with 264
    (8, 2, (1, 0), ((2500, 8300), (6000, 8000)), -1),
    (8, 2, (1, 0), ((2500, 8300), (6000, 8000)), 24),
    (8, 2, (1, 0), ((0, 8256),), -1),
    (8, 8, (1, 0, 0, 0, 0, 0, 0, 1), ((1000, 8448),), -1),
    (16, 2, (0, 1), ((3000, 4200),), 32),
]


@pytest.mark.parametrize("case", PERSISTENT, ids=["g4_whole", "g4_split", "g4_cus_plus_2", "g1", "g8_split"])
def test_persistent_queues_sampled(case):
    """More 256-pair units than CUs: the two-block kernel runs persistent, one
    workgroup per CU taking the other units from its XCD's queue and, at the
    end, from the other XCDs' queues. A global and a local head of unequal
    unit costs, with and without split runs: sampled rows (band edges, page
    edges, uniform) against the oracle, bf16 output = RNE(fp32), and a rerun
    bitwise identical (which workgroup runs a unit does not change its
    result)."""
    hq, hkv, classes, seqs, run = case
    w = adhoc(hq=hq, hkv=hkv, d=128, page=64, window=1500, classes=classes, seqs=seqs, seed=41 + run + len(seqs) + hq)
    o, lse, gl = run_case(w, queries="sampled", seed=abs(run), max_unit_tiles=run)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert gl.host["unit_rows"] * gl.host["unit_heads"] == 256 and gl.host["num_units"] > cus
    assert (gl.host["num_parts"] > 0) == (run > 0)
    ob, _ = gl.attention(torch.bfloat16, with_lse=False)
    o2, l2 = gl.attention(torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(ob, o.to(torch.bfloat16))
    assert torch.equal(o2, o) and torch.equal(l2, lse)


DECODE = [
    # (hq, hkv, d, page, window, classes, seqs, longest run in tiles: 0 automatic)
    (8, 2, 128, 64, 100, (0, 1), ((300, 1), (37, 5), (1000, 8), (5, 3)), 0),
    (16, 2, 64, 128, 300, (1, 0), ((250, 2), (0, 4), (700, 1)), 3),
    (8, 1, 128, 256, 40, (0,), ((700, 4), (3, 1)), 1),
    (4, 4, 64, 64, 1, (1, 1, 0, 0), ((130, 7), (64, 32), (0, 1)), 2),
    (32, 2, 128, 64, 2000, (1, 0), ((3000, 1), (64, 2)), 5),
    (6, 3, 128, 64, 17, (0, 1, 0), ((129, 16), (500, 9)), 0),
]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: f"hq{c[0]}_kv{c[1]}_d{c[2]}_p{c[3]}_run{c[7]}")
def test_decode_units_all_rows(case):
    """A few new rows per sequence (at most 32 / G): decode units, one (row,
    head) pair per MFMA column, with and without split runs."""
    hq, hkv, d, page, window, classes, seqs, run = case
    w = adhoc(hq=hq, hkv=hkv, d=d, page=page, window=window, classes=classes, seqs=seqs, seed=hq + d + run)
    o, lse, gl = run_case(w, max_unit_tiles=run)
    G = hq // hkv
    assert (gl.host["unit_rows"], gl.host["unit_heads"]) == (32 // G, G)
    ob, _ = gl.attention(torch.bfloat16, with_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(ob, o.to(torch.bfloat16))


def test_decode_32k_all_rows():
    """One decode step of 32 sequences at 32K (one new row each): every row of
    every head against the oracle, split-KV runs merged."""
    o, lse, gl = run_case(DECODE_32K)
    assert gl.host["num_parts"] > 0


def test_mistral_8k_all_rows():
    """The 8K layer, every row of every head (about 3.5e8 visible pairs for
    the oracle); split automatically (its longest block exceeds the mean load
    per workgroup slot)."""
    o, lse, gl = run_case(MISTRAL_8K, queries="all")
    assert gl.host["num_parts"] > 0


def test_llama70b_32k_sampled():
    run_case(LLAMA70B_32K, queries="sampled", seed=3)


def test_varlen_chunked_all_rows():
    """16 sequences, 2048-row chunks over cached prefixes: every row of every
    head (about 3.4e9 visible pairs for the oracle); then the bf16 output
    equals the fp32 output rounded to nearest even."""
    o, lse, gl = run_case(VARLEN_CHUNKED, queries="all")
    ob, _ = gl.attention(torch.bfloat16, with_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(ob, o.to(torch.bfloat16))


def _stack_layers():
    """Two layers of every class of the 128K stack (0, 1, 2 and 3 global KV
    heads: the first two of each), or all 64 with SEGKV_FULL_STACK=1."""
    r = realize(STACK64_128K)
    g = r.head_class.sum(axis=1)
    if os.environ.get("SEGKV_FULL_STACK") == "1":
        return list(range(STACK64_128K.layers))
    pick = []
    for c in sorted(set(g.tolist())):
        pick += [int(i) for i in np.nonzero(g == c)[0][:2]]
    return sorted(pick)


_STACK_G = realize(STACK64_128K).head_class.sum(axis=1)


@pytest.mark.parametrize("layer", _stack_layers(), ids=lambda l: f"layer{l}_g{int(_STACK_G[l])}")
def test_stack128k_sampled_layer(layer):
    """One layer of the 64-layer 128K stack, sampled rows of every head (256
    seeded-uniform rows per head plus the first/last, window-edge and
    page-boundary rows), fp32 output against the oracle; then the bf16
    output the bench times (same kernel, bf16 store) equals the fp32 output
    rounded to nearest even, bit for bit."""
    w = STACK64_128K
    r = realize(w)
    pools = device_pools(r.num_pages, w.page, w.d)
    say(f"[case] {w.name} layer {layer} globals {int(r.head_class[layer].sum())}")
    t = layer_tensors(w, r, layer, device="cuda")
    gl = GpuLayer(w, r, layer, t, pools=pools)
    o, lse = gl.run(torch.float32)
    ob, _ = gl.attention(torch.bfloat16, with_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(ob, o.to(torch.bfloat16))
    bits = {k: host_bits(v) for k, v in t.items()}
    del t, gl, ob
    q = sampled_queries(w, r, layer, seed=100 + layer, n_uniform=256)
    oo, ol, tab = oracle_queries(w, r, layer, bits, q)
    stats = compare(o, lse, oo, ol, q, tab, w.hkv)
    say(f"[ok] {w.name} layer {layer}: {stats}")
    del o, lse, bits
    torch.cuda.empty_cache()


@pytest.mark.parametrize("w", [TINY, adhoc(hq=8, hkv=2, d=128, page=64, window=100, classes=(0, 1),
                                            seqs=((0, 200), (37, 301)), seed=9),
                               adhoc(hq=8, hkv=2, d=128, page=64, window=1500, classes=(1, 0),
                                     seqs=((2500, 333),), seed=19)],
                         ids=["tiny", "ragged", "wide_g4"])
def test_bitwise_invariances(w):
    r = realize(w)
    t = layer_tensors(w, r, 0, device="cuda")
    base_o, base_l = GpuLayer(w, r, 0, t).run()
    # rerun
    o2, l2 = GpuLayer(w, r, 0, t).run()
    assert torch.equal(base_o, o2) and torch.equal(base_l, l2)
    # physical page relabelling
    po = relabel_pages(r.page_of, r.num_pages, 77)[0]
    o3, l3 = GpuLayer(w, r, 0, t, page_of=po).run()
    assert torch.equal(base_o, o3) and torch.equal(base_l, l3)
    # NaN in every slot that is never written (free pages, page tails)
    o4, l4 = GpuLayer(w, r, 0, t, poison=True).run()
    assert torch.equal(base_o, o4) and torch.equal(base_l, l4)


def test_write_gather_roundtrip_bit_exact():
    import head_segmented_paged_amd as H
    w = adhoc(hq=4, hkv=2, d=128, page=16, window=20, classes=(1, 0), seqs=((37, 100), (0, 5), (16, 16)), seed=4)
    r = realize(w)
    t = layer_tensors(w, r, 0, device="cuda")
    gl = GpuLayer(w, r, 0, t, poison=True)
    gl.write()
    torch.cuda.synchronize()
    bits = {k: host_bits(v) for k, v in t.items()}
    kp, vp = opaged.empty_pools(r.num_pages, w.page, w.d)
    written = np.zeros(r.num_pages, bool)
    opaged.scatter_pages(kp, vp, r.page_of[0], r.cached_len, r.new_len, bits["k_cached"], bits["v_cached"],
                         bits["k_new"], bits["v_new"])
    ids = np.unique(r.page_of[0][r.page_of[0] >= 0]).astype(np.int32)
    written[ids] = True
    dev_ids = torch.from_numpy(ids).cuda()
    ko = torch.empty((len(ids), w.page, w.d), dtype=torch.bfloat16, device="cuda")
    vo = torch.empty_like(ko)
    H.segkv_gather_pages(gl.ctx, dev_ids, ko, vo)
    torch.cuda.synchronize()
    kg, vg = host_bits(ko), host_bits(vo)
    # every slot of a sequence's positions matches the oracle's scatter bit for bit
    for b in range(r.num_seqs):
        T = int(r.cached_len[b] + r.new_len[b])
        for g in range(w.hkv):
            for p in range(T):
                pid = r.page_of[0][b, g, p // w.page]
                i = np.searchsorted(ids, pid)
                assert np.array_equal(kg[i, p % w.page], kp[pid, p % w.page])
                assert np.array_equal(vg[i, p % w.page], vp[pid, :, p % w.page])
    # free pages are untouched (still NaN)
    free = np.nonzero(~written)[0][:64]
    assert torch.isnan(gl.k_pool[torch.from_numpy(free).cuda()].float()).all()
    assert torch.isnan(gl.v_pool[torch.from_numpy(free).cuda()].float()).all()
