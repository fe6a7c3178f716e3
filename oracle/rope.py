"""Oracle for RoPE re-alignment of reused K rows (test infrastructure only:
used by tests/ and nothing else; shares no code with the library).

RedKnot summary page, "Elastic Sparsity": recovering a reused (position-
independent) KV segment starts by aligning RoPE positions. A K row stored
with rotary angles for position p must read as the row for position
p + delta. Rotary embedding turns each pair of dimensions by an angle
proportional to the position, and turns add, so the re-aligned row is the
stored row turned once more by delta * theta_i.

Reading taken (the pages fix neither): pairs are (i, i + D/2) for i < D/2
("rotate half"), theta_i = base^(-2 i / D), base 10000 unless given; the
rotation is counter-clockwise, x' = x cos a - y sin a, y' = x sin a + y cos a.
Everything is fp64; the result is rounded to bf16 (nearest even) because the
pages store K in bf16.
"""

import numpy as np


def angles(D, delta, base=10000.0):
    """a_i = delta * base^(-2 i / D), i < D / 2, in fp64."""
    i = np.arange(D // 2, dtype=np.float64)
    return float(delta) * np.power(float(base), -2.0 * i / D)


def rotate(k, delta, base=10000.0):
    """k: float64 [..., D] rows encoded at position p -> rows encoded at p + delta (fp64)."""
    k = np.asarray(k, dtype=np.float64)
    D = k.shape[-1]
    a = angles(D, delta, base)
    c, s = np.cos(a), np.sin(a)
    x, y = k[..., : D // 2], k[..., D // 2:]
    return np.concatenate([x * c - y * s, x * s + y * c], axis=-1)


def encode(k, pos, base=10000.0):
    """Rotary encoding of raw rows k [n][D] at positions pos [n] (the same turn as rotate)."""
    k = np.asarray(k, dtype=np.float64)
    return np.stack([rotate(k[j], int(pos[j]), base) for j in range(k.shape[0])])


def to_bf16_bits(x):
    """fp64 -> bf16 bit patterns, rounded once to 8 significant bits, ties to
    even (normal range; the stored values are far from under- or overflow)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                                  # x = m 2^e, |m| in [0.5, 1)
    r = np.ldexp(np.rint(m * 256.0), e - 8)             # np.rint: ties to even
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def realign_pages(k_pool_bits, entries, base=10000.0):
    """Reference for segkv_rope_realign on a host copy of the K pool.
    k_pool_bits: uint16 [num_pages][P][D] (bf16 bits), entries int [n][4] =
    (page, slot0, nslots, delta). Returns a new uint16 pool."""
    out = np.array(k_pool_bits, copy=True)
    num_pages, P, _ = out.shape
    for page, slot0, nslots, delta in np.asarray(entries, dtype=np.int64):
        if page < 0 or page >= num_pages or slot0 < 0 or slot0 >= P or nslots <= 0:
            continue
        s1 = slot0 + min(nslots, P - slot0)
        rows = bf16_bits_to_f64(out[page, slot0:s1])
        out[page, slot0:s1] = to_bf16_bits(rotate(rows, delta, base))
    return out
