"""Pins for the fp64 attention oracle (CPU only).

The oracle is checked against things other than itself:
  * brute force: dense float64 attention with an explicit boolean mask built
    element by element (oracle/bruteforce.py), on the tiny workload and on a
    sweep of small shapes with ragged lengths, windows around the page size
    and cached prefixes;
  * closed forms: the first query of a sequence returns v_0 exactly; W = 1
    returns v_i exactly; Q = 0 returns the plain mean of exactly the visible
    value rows; constant V returns the constant;
  * a library routine: for a global head with no cached prefix the result is
    torch's float64 causal scaled_dot_product_attention;
  * invariants: a local head whose window covers the whole sequence equals a
    global head bit for bit; relabelling physical pages changes nothing bit
    for bit; a chunk (c, n) equals rows c..c+n-1 of a monolithic prefill.
"""

import numpy as np
import pytest
import torch

from oracle import bruteforce
from oracle import paged as opaged
from tests.common import adhoc, bits_to_f64, make_case, oracle_all
from workloads import TINY


def _windows(case):
    return np.where(case.head_class == 1, 0, case.w.window)


def brute(case):
    ks, vs = case.dense_kv()
    return bruteforce.layer_reference(bits_to_f64(case.bits["q"]), ks, vs, case.cached_len, case.new_len,
                                      case.head_class, _windows(case), case.w.hq, case.w.hkv, case.scale)


def test_tiny_workload_matches_bruteforce():
    case = make_case(TINY)
    O, L = oracle_all(case)
    Ob, Lb = brute(case)
    assert np.isfinite(O).all()
    assert np.max(np.abs(O - Ob)) <= 1e-12
    assert np.max(np.abs(L - Lb)) <= 1e-12


SWEEP = []
for L in (1, 2, 15, 16, 17, 100):
    for W in (1, 2, 15, 16, 17, L - 1, L, L + 7):
        for c in (0, 5, 37):
            if W >= 1:
                SWEEP.append((L, W, c))
SWEEP = sorted(set(SWEEP))


@pytest.mark.parametrize("L,W,c", SWEEP)
def test_sweep_matches_bruteforce(L, W, c):
    # two sequences (the second short), hkv 2 with one global and one local head, G = 2
    w = adhoc(hq=4, hkv=2, d=8, page=16, window=W, classes=(0, 1), seqs=((c, L), (3, 7)),
              seed=100 + L * 1000 + W * 10 + c)
    case = make_case(w)
    O, Lo = oracle_all(case)
    Ob, Lb = brute(case)
    assert np.max(np.abs(O - Ob)) <= 1e-12
    assert np.max(np.abs(Lo - Lb)) <= 1e-12


def test_first_query_returns_first_value_exactly():
    case = make_case(adhoc(d=16, window=5, seqs=((0, 30), (0, 3))))
    O, _ = oracle_all(case)
    ks, vs = case.dense_kv()
    G = case.w.hq // case.w.hkv
    for h in range(case.w.hq):
        assert np.array_equal(O[0, h], vs[0][0, h // G])
        assert np.array_equal(O[30, h], vs[1][0, h // G])


def test_window_one_returns_own_value_exactly():
    case = make_case(adhoc(d=16, window=1, classes=(0, 0), seqs=((11, 40),)))
    O, _ = oracle_all(case)
    _, vs = case.dense_kv()
    G = case.w.hq // case.w.hkv
    for t in range(40):
        for h in range(case.w.hq):
            assert np.array_equal(O[t, h], vs[0][11 + t, h // G])


@pytest.mark.parametrize("W", [1, 3, 16, 17, 50])
def test_zero_query_gives_mean_of_exactly_the_visible_rows(W):
    case = make_case(adhoc(d=16, window=W, classes=(1, 0), seqs=((9, 45),)), build=False)
    case.bits["q"] = np.zeros_like(case.bits["q"])
    from tests.common import build_oracle_state
    build_oracle_state(case)
    O, Lse = oracle_all(case)
    _, vs = case.dense_kv()
    for t in range(45):
        i = 9 + t
        glob = vs[0][: i + 1].mean(axis=0)            # kv head 0: global
        loc = vs[0][max(0, i - W + 1): i + 1].mean(axis=0)  # kv head 1: the W newest keys incl. self
        np.testing.assert_allclose(O[t, 0], glob[0], atol=1e-12, rtol=0)
        np.testing.assert_allclose(O[t, 2], loc[1], atol=1e-12, rtol=0)
        np.testing.assert_allclose(Lse[t, 2], np.log(min(i + 1, W)), atol=1e-12, rtol=0)


def test_constant_values_give_the_constant():
    case = make_case(adhoc(d=16, window=6, seqs=((4, 33),)), build=False)
    for key in ("v_new", "v_cached"):
        case.bits[key] = np.full_like(case.bits[key], 0x3FC0)   # bf16 1.5
    from tests.common import build_oracle_state
    build_oracle_state(case)
    O, _ = oracle_all(case)
    np.testing.assert_allclose(O, 1.5, atol=1e-13, rtol=0)


def test_global_head_equals_torch_causal_sdpa():
    case = make_case(adhoc(hq=4, hkv=2, d=32, page=16, classes=(1, 1), seqs=((0, 77),)))
    O, _ = oracle_all(case)
    ks, vs = case.dense_kv()
    q = torch.from_numpy(bits_to_f64(case.bits["q"]))            # [77][4][32]
    G = 2
    for h in range(4):
        k = torch.from_numpy(ks[0][:, h // G, :])
        v = torch.from_numpy(vs[0][:, h // G, :])
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[:, h, :][None], k[None], v[None], is_causal=True).numpy()[0]
        np.testing.assert_allclose(O[:, h, :], ref, atol=1e-12, rtol=0)


def test_window_covering_sequence_equals_global_bitwise():
    base = dict(hq=4, hkv=2, d=16, page=16, seqs=((0, 50), (13, 20)), seed=5)
    glob = make_case(adhoc(classes=(1, 1), window=8, **base))
    loc = make_case(adhoc(classes=(0, 0), window=33 + 20 + 7, **base))
    Og, Lg = oracle_all(glob)
    Ol, Ll = oracle_all(loc)
    assert np.array_equal(Og, Ol) and np.array_equal(Lg, Ll)


def test_page_relabelling_is_bitwise_invariant():
    w = adhoc(hq=4, hkv=2, d=16, page=16, window=19, seqs=((21, 60), (0, 17)))
    a = make_case(w)
    b = make_case(w, relabel_seed=99)
    assert not np.array_equal(a.page_of, b.page_of)
    Oa, La = oracle_all(a)
    Ob, Lb = oracle_all(b)
    assert np.array_equal(Oa, Ob) and np.array_equal(La, Lb)


@pytest.mark.parametrize("W,classes", [(10, (0, 1)), (64, (0, 0))])
def test_chunk_equals_monolithic(W, classes):
    c, n = 37, 63
    mono = make_case(adhoc(hq=4, hkv=2, d=16, page=16, window=W, classes=classes, seqs=((0, c + n),), seed=3))
    bits = mono.bits
    chunk_bits = {
        "q": bits["q"][c:], "k_new": bits["k_new"][c:], "v_new": bits["v_new"][c:],
        "k_cached": bits["k_new"][:c], "v_cached": bits["v_new"][:c],
    }
    chunk = make_case(adhoc(hq=4, hkv=2, d=16, page=16, window=W, classes=classes, seqs=((c, n),), seed=3),
                      bits=chunk_bits)
    Om, Lm = oracle_all(mono)
    Oc, Lc = oracle_all(chunk)
    assert np.array_equal(Om[c:], Oc) and np.array_equal(Lm[c:], Lc)


def test_bad_page_list_is_reported():
    case = make_case(adhoc(seqs=((0, 40),)))
    q = opaged.all_queries(case.tables, case.w.hq)
    t = dict(case.tables)
    t["page_list"] = t["page_list"].copy()
    t["page_list"][0] = case.num_pages + 5
    with pytest.raises(ValueError):
        opaged.attention(case.k_pool, case.v_pool, case.bits["q"], t, q)
