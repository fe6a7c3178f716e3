"""Pins of the oracle's attention mass (oracle_mass_fp64): the weight each new
token receives, summed over every query row and query head of the step.

Pinned against: brute-force column sums of explicitly masked dense softmax
matrices; the closed form for Q = 0 (uniform attention over the visible
keys: token j gets sum over the rows i that see it of 1 / |V(i)|); and the
total (with no cached prefix every query's weights sum to one over new
tokens, so the masses add up to rows x heads)."""

import numpy as np
import pytest

from oracle import bruteforce
from oracle import paged as opaged
from tests.common import adhoc, bits_to_f64, make_case


def _mass(case):
    q = opaged.all_queries(case.tables, case.w.hq)
    return opaged.attention_mass(case.k_pool, case.bits["q"], case.tables, q)


def _brute_mass(case):
    w, t = case.w, case.tables
    G = w.hq // w.hkv
    D = w.d
    q = bits_to_f64(case.bits["q"])
    kc, kn = bits_to_f64(case.bits["k_cached"]), bits_to_f64(case.bits["k_new"])
    out = np.zeros(q.shape[0])
    c_off, n_off = 0, 0
    for b in range(len(case.cached_len)):
        c, n = int(case.cached_len[b]), int(case.new_len[b])
        for h in range(w.hq):
            g = h // G
            k = np.concatenate([kc[c_off:c_off + c, g], kn[n_off:n_off + n, g]])      # dense logical K
            glob = bool(case.head_class[g])
            M = bruteforce.visibility_mask(c, n, glob, int(case.window[g]))
            S = (q[n_off:n_off + n, h] @ k.T) / np.sqrt(D)
            S[~M] = -np.inf
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            out[n_off:n_off + n] += P[:, c:].sum(axis=0)
        c_off += c
        n_off += n
    return out


CASES = [
    dict(hq=4, hkv=2, d=16, page=16, window=8, classes=(1, 0), seqs=((0, 40),)),
    dict(hq=6, hkv=3, d=8, page=4, window=5, classes=(0, 1, 0), seqs=((7, 13), (0, 9), (30, 2))),
    dict(hq=2, hkv=1, d=32, page=16, window=1, classes=(0,), seqs=((3, 20),)),
    dict(hq=8, hkv=2, d=16, page=8, window=100, classes=(0, 0), seqs=((50, 30),)),
]


@pytest.mark.parametrize("kw", CASES)
def test_mass_matches_bruteforce(kw):
    case = make_case(adhoc(seed=11, **kw))
    np.testing.assert_allclose(_mass(case), _brute_mass(case), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("W", [1, 3, 8, 64])
def test_mass_zero_query_closed_form(W):
    w = adhoc(hq=4, hkv=2, d=16, page=8, window=W, classes=(1, 0), seqs=((5, 30),), seed=3)
    case = make_case(w, build=False)
    case.bits["q"] = np.zeros_like(case.bits["q"])
    from tests.common import build_oracle_state
    build_oracle_state(case)
    got = _mass(case)
    c, n = 5, 30
    expect = np.zeros(n)
    for g, glob in enumerate((1, 0)):
        for t in range(n):
            i = c + t
            lo = 0 if glob else max(0, i - W + 1)
            for j in range(max(lo, c), i + 1):
                expect[j - c] += 2 * (1.0 / (i - lo + 1))          # two query heads per KV head
    np.testing.assert_allclose(got, expect, rtol=1e-12)


def test_mass_total_without_cache():
    case = make_case(adhoc(hq=8, hkv=4, d=16, page=16, window=7, classes=(1, 0, 0, 1),
                           seqs=((0, 50), (0, 17)), seed=5))
    assert np.isclose(_mass(case).sum(), 8 * 67, rtol=1e-12)
