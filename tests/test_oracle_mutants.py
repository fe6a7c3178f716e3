"""The oracle's pins catch plausible mistakes (CPU only).

Each case below copies oracle/attn_fp64.c to a temporary directory, plants
one plausible mistake in the copy (a window off by one, a strict causal
compare, a transposed value index, a dropped scale, a wrong GQA mapping, a
page index without the segment's first page, a flipped max subtraction, a
dropped term in the log-sum-exp), compiles it, and runs a battery of the
same checks the pin tests use. The real oracle must pass the battery and
every mutant must fail at least one check.
"""

import os
import tempfile

import numpy as np
import pytest

from oracle import bruteforce
from oracle import paged as opaged
from tests.common import adhoc, bits_to_f64, build_oracle_state, make_case, oracle_all

SRC = os.path.join(os.path.dirname(opaged.__file__), "attn_fp64.c")

MUTANTS = {
    "window_off_by_one": ("i - window[s] + 1 > 0 ? i - window[s] + 1", "i - window[s] > 0 ? i - window[s]"),
    "strict_causal": ("for (int64_t j = lo; j <= i; ++j) {\n            int64_t e", "for (int64_t j = lo; j < i; ++j) {\n            int64_t e"),
    "transposed_v": ("vpage[(int64_t)d * P + j % P]", "vpage[(int64_t)(j % P) * D + d]"),
    "dropped_scale": ("score[j - lo] = scale * dot;", "score[j - lo] = dot;"),
    "gqa_modulo": ("const int32_t g = h / G;", "const int32_t g = h % hkv;"),
    "page_index_absolute": ("int64_t e = (int64_t)cu_pages[s] + (j / P - first_lp);",
                            "int64_t e = (int64_t)cu_pages[s] + (j / P);"),
    "flipped_max": ("double p = exp(score[j - lo] - m);", "double p = exp(m - score[j - lo]);"),
    "lse_drops_max": ("lse[x] = m + log(denom);", "lse[x] = log(denom);"),
}


def _battery(lib_path):
    """Return the list of failed checks for the oracle library at lib_path."""
    failed = []

    def run(case):
        try:
            return oracle_all(case, lib_path=lib_path)
        except ValueError:
            return None

    def brute(case):
        ks, vs = case.dense_kv()
        win = np.where(case.head_class == 1, 0, case.w.window)
        return bruteforce.layer_reference(bits_to_f64(case.bits["q"]), ks, vs, case.cached_len, case.new_len,
                                          case.head_class, win, case.w.hq, case.w.hkv, case.scale)

    # brute force on a multi-sequence case with cached prefixes and both classes
    for W in (5, 16, 17):
        case = make_case(adhoc(hq=4, hkv=2, d=8, page=16, window=W, classes=(0, 1),
                               seqs=((37, 40), (0, 21)), seed=W))
        res = run(case)
        if res is None:
            failed.append(f"bruteforce W={W}: oracle error")
            continue
        O, L = res
        Ob, Lb = brute(case)
        if not (np.nanmax(np.abs(O - Ob)) <= 1e-12) or not np.isfinite(O).all():
            failed.append(f"bruteforce W={W}: O")
        if not (np.nanmax(np.abs(L - Lb)) <= 1e-12):
            failed.append(f"bruteforce W={W}: lse")

    # Q = 0: mean of exactly the visible rows
    case = make_case(adhoc(d=8, window=6, classes=(1, 0), seqs=((9, 30),)), build=False)
    case.bits["q"] = np.zeros_like(case.bits["q"])
    build_oracle_state(case)
    res = run(case)
    _, vs = case.dense_kv()
    if res is None:
        failed.append("zero-q: oracle error")
    else:
        O, _ = res
        for t in range(30):
            i = 9 + t
            if not np.allclose(O[t, 2], vs[0][max(0, i - 5): i + 1, 1].mean(axis=0), atol=1e-12, rtol=0):
                failed.append("zero-q mean")
                break
    return failed


def _compile_mutant(name, tmp):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    path = os.path.join(tmp, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    return opaged.build(src=path, out=os.path.join(tmp, f"lib_{name}.so"))


def test_real_oracle_passes_battery():
    assert _battery(opaged.load() and opaged._LIB) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    with tempfile.TemporaryDirectory() as tmp:
        lib = _compile_mutant(name, tmp)
        failed = _battery(lib)
    assert failed, f"mutant {name} passed every pin"
