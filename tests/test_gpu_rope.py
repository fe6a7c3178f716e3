"""GPU parity of the RoPE re-alignment of reused K pages against the fp64
oracle (oracle/rope.py), through the C ABI.

Bar: rotated elements equal the oracle's bf16 (nearest even of the exact
rotation) except for at most 1 ulp on at most 0.1 % of them. The kernel
rounds the fp64 cos/sin to fp32 and rotates in fp32 (relative error about
3e-7), so it can only disagree where the exact value lies within that distance
of a bf16 rounding midpoint (probability about 2 * 3e-7 / 2^-8 = 1.5e-4).
Everything not named by an entry (other slots, other pages, all of V) is
unchanged bit for bit."""

import numpy as np
import pytest
import torch

import head_segmented_paged_amd as H
from oracle import rope
from tests.gpu_helpers import say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("D,P,base", [(128, 64, 10000.0), (64, 16, 500000.0), (128, 256, 10000.0)])
def test_rope_realign_matches_oracle(D, P, base):
    say(f"[case] rope D {D} P {P} base {base}")
    num_pages = 40
    g = torch.Generator(device="cpu").manual_seed(D + P)
    k = torch.randn((num_pages, P, D), generator=g).to(torch.bfloat16)
    v = torch.randn((num_pages, D, P), generator=g).to(torch.bfloat16)
    kd, vd = k.cuda(), v.cuda()
    ctx = H.segkv_create(kd, vd, 8, 2, D, P)
    entries = [(p, 0, P, d) for p, d in zip(range(0, 20), (1, -1, 7, 1000, 131071, -65536, 1 << 20, 3, 0, 5,
                                                          -7, 2048, 4095, 99, 100000, -1, 12, 13, 14, 15))]
    entries += [(21, 5, 10, 333), (22, P - 4, 100, -1234), (23, 0, 1, 77)]
    entries += [(-1, 0, P, 5), (num_pages, 0, P, 5), (24, P, 4, 5), (25, 0, 0, 5), (26, -3, 4, 5)]
    ent = torch.tensor(entries, dtype=torch.int32).cuda()
    H.segkv_rope_realign(ctx, ent, base)
    torch.cuda.synchronize()
    got = kd.cpu().view(torch.int16).numpy().view(np.uint16)
    before = k.view(torch.int16).numpy().view(np.uint16)
    expect = rope.realign_pages(before, entries, base)
    touched = np.zeros_like(got, dtype=bool)
    for p, s0, n, _ in entries:
        if 0 <= p < num_pages and 0 <= s0 < P and n > 0:
            touched[p, s0:s0 + min(n, P - s0)] = True
    assert np.array_equal(got[~touched], before[~touched])
    diff = np.abs(got[touched].astype(np.int32) - expect[touched].astype(np.int32))
    # same sign, so bit patterns one apart are one ulp apart
    assert diff.max() <= 1
    frac = (diff > 0).mean()
    say(f"[ok] rope D {D} P {P}: {touched.sum()} rotated values, {frac:.2e} one ulp off")
    assert frac <= 1e-3
    assert torch.equal(vd.cpu(), v)
