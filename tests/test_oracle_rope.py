"""Pins of the RoPE re-alignment oracle (oracle/rope.py) against facts the
definition fixes: the zero turn, composition of turns, norm preservation, the
relative-position property of rotary scores, a hand-computed D = 4 example of
the pairing, and nearest-even rounding to bf16."""

import math

import numpy as np
import pytest
import torch

from oracle import rope


def _rows(n, D, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal((n, D))


def test_zero_turn_is_identity():
    k = _rows(7, 128, 1)
    assert np.array_equal(rope.rotate(k, 0), k)


@pytest.mark.parametrize("a,b", [(1, 2), (-5, 17), (1000, -999), (123456, 65536)])
def test_turns_compose(a, b):
    k = _rows(5, 64, 2)
    np.testing.assert_allclose(rope.rotate(rope.rotate(k, a), b), rope.rotate(k, a + b), rtol=0, atol=1e-9)


def test_pair_norms_preserved():
    k = _rows(9, 128, 3)
    r = rope.rotate(k, 4321)
    n0 = k[:, :64] ** 2 + k[:, 64:] ** 2
    n1 = r[:, :64] ** 2 + r[:, 64:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)


def test_scores_depend_on_relative_position_only():
    q, k = _rows(1, 128, 4), _rows(1, 128, 5)
    for p, pk, shift in ((10, 3, 100), (0, 0, 77777), (5000, 4000, -4000)):
        s0 = rope.encode(q, [p]) @ rope.encode(k, [pk]).T
        s1 = rope.encode(q, [p + shift]) @ rope.encode(k, [pk + shift]).T
        np.testing.assert_allclose(s1, s0, rtol=1e-9)
    # and re-aligning a stored key by delta equals encoding it at the new position
    raw = _rows(3, 128, 6)
    np.testing.assert_allclose(rope.rotate(rope.encode(raw, [1, 2, 3]), 50), rope.encode(raw, [51, 52, 53]),
                               atol=1e-10)


def test_pairing_by_hand():
    """D = 4, base 100: theta = (1, 0.1); pairs (0, 2) and (1, 3), turned counter-clockwise."""
    k = np.array([1.0, 2.0, 0.5, -1.0])
    c1, s1 = math.cos(3.0), math.sin(3.0)        # pair (0, 2): angle 3 * 1
    c2, s2 = math.cos(0.3), math.sin(0.3)        # pair (1, 3): angle 3 * 0.1
    expect = [1.0 * c1 - 0.5 * s1, 2.0 * c2 - (-1.0) * s2, 1.0 * s1 + 0.5 * c1, 2.0 * s2 + (-1.0) * c2]
    np.testing.assert_allclose(rope.rotate(k, 3, base=100.0), expect, rtol=0, atol=1e-15)


def test_bf16_rounding_nearest_even():
    x = np.random.Generator(np.random.PCG64(7)).standard_normal(10000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(rope.to_bf16_bits(x.astype(np.float64)), ref)
    # exact ties between neighbours go to the even significand
    one_ulp = 2.0 ** -7                           # bf16 spacing in [1, 2)
    ties = np.array([1.0 + 0.5 * one_ulp, 1.0 + 1.5 * one_ulp, -(1.0 + 2.5 * one_ulp)])
    got = rope.bf16_bits_to_f64(rope.to_bf16_bits(ties))
    np.testing.assert_array_equal(got, [1.0, 1.0 + 2 * one_ulp, -(1.0 + 2 * one_ulp)])
    # a value just above a tie (below fp32 resolution of the tie) rounds up: no double rounding
    assert rope.bf16_bits_to_f64(rope.to_bf16_bits(np.array([1.0 + 0.5 * one_ulp + 2.0 ** -40])))[0] == 1.0 + one_ulp


def test_realign_pages_skips_bad_entries_and_cuts_at_page_end():
    rng = np.random.Generator(np.random.PCG64(8))
    pool = rope.to_bf16_bits(rng.standard_normal((4, 16, 8)))
    ent = [(1, 3, 100, 5), (7, 0, 4, 1), (-1, 0, 4, 1), (2, 16, 4, 1), (3, 0, 0, 9)]
    out = rope.realign_pages(pool, ent)
    assert np.array_equal(out[[0, 2, 3]], pool[[0, 2, 3]])
    assert np.array_equal(out[1, :3], pool[1, :3])
    expect = rope.to_bf16_bits(rope.rotate(rope.bf16_bits_to_f64(pool[1, 3:]), 5))
    assert np.array_equal(out[1, 3:], expect)
