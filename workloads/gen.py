"""Seeded synthetic inputs for head-segmented paged prefill.

Everything here is input preparation, shared by the tests, the benchmark and
the smoke check: the head-class table, the sequence lengths, the block
(page) table that maps each (layer, sequence, KV head, logical page) to a
physical page of one shared pool, and bf16 N(0, 1) tensors for Q and for the
cached and new K/V rows. None of the method's arithmetic lives here: which
pages a head reads, the visible sets and the attention itself are computed by
the library under test and, independently, by the oracle.

Block tables follow the PagedAttention idea summarised on the KV-cache
management page (section 3.1: fixed-size blocks, logical-to-physical
mapping): every logical page of every (layer, sequence, KV head) gets a
physical id from a seeded permutation of the pool, so neighbouring logical
pages land on unrelated physical pages.
"""

from dataclasses import dataclass

import numpy as np

from .configs import Workload


@dataclass
class Realized:
    """One concrete draw of a workload's metadata (host arrays)."""
    w: Workload
    cached_len: np.ndarray   # int32 [S]   c_b
    new_len: np.ndarray      # int32 [S]   n_b
    head_class: np.ndarray   # int8  [layers][hkv]   1 = global, 0 = local
    window: np.ndarray       # int32 [layers][hkv]   W for local heads, 0 for global
    page_of: np.ndarray      # int32 [layers][S][hkv][max_lp]   -1 = no page
    num_pages: int           # pool capacity

    @property
    def num_seqs(self) -> int:
        return int(self.cached_len.shape[0])

    @property
    def max_lp(self) -> int:
        return int(self.page_of.shape[-1])

    @property
    def total_len(self) -> np.ndarray:
        return (self.cached_len.astype(np.int64) + self.new_len).astype(np.int32)


def _rng(seed: int, *tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *tag])))


def draw_classes(w: Workload) -> np.ndarray:
    rule = w.class_rule
    cls = np.zeros((w.layers, w.hkv), dtype=np.int8)
    if rule[0] == "fixed":
        cls[:] = np.asarray(rule[1], dtype=np.int8)
    elif rule[0] == "count":
        k = int(rule[1])
        rng = _rng(w.seed, 1)
        for layer in range(w.layers):
            cls[layer, rng.choice(w.hkv, size=k, replace=False)] = 1
    elif rule[0] == "bernoulli":
        p, first_free = float(rule[1]), int(rule[2])
        rng = _rng(w.seed, 1)
        draws = rng.random((w.layers, w.hkv))
        cls[:] = (draws < p).astype(np.int8)
        cls[:first_free] = 0
    else:
        raise ValueError(f"unknown class rule {rule!r}")
    return cls


def draw_seqs(w: Workload):
    rule = w.seq_rule
    if rule[0] == "fixed":
        c = np.array([s[0] for s in rule[1]], dtype=np.int32)
        n = np.array([s[1] for s in rule[1]], dtype=np.int32)
    elif rule[0] == "uniform_cached":
        nseq, lo, hi, n_new = (int(x) for x in rule[1:])
        rng = _rng(w.seed, 2)
        c = rng.integers(lo, hi + 1, size=nseq).astype(np.int32)
        n = np.full(nseq, n_new, dtype=np.int32)
    else:
        raise ValueError(f"unknown sequence rule {rule!r}")
    return c, n


def allocate_pages(layers: int, hkv: int, page: int, total_len: np.ndarray,
                   seed: int, slack: float = 1.25):
    """Give every logical page of every (layer, sequence, KV head) a physical
    page id from a seeded permutation of a pool of ceil(slack * needed) pages.
    Returns (page_of [layers][S][hkv][max_lp] int32, num_pages)."""
    lp_count = (total_len.astype(np.int64) + page - 1) // page          # [S]
    max_lp = int(lp_count.max()) if lp_count.size else 0
    need = int(layers * hkv * lp_count.sum())
    num_pages = max(int(np.ceil(need * slack)), need + 1)
    perm = _rng(seed, 3).permutation(num_pages).astype(np.int32)
    page_of = np.full((layers, total_len.shape[0], hkv, max(max_lp, 1)), -1, dtype=np.int32)
    cursor = 0
    for layer in range(layers):
        for b in range(total_len.shape[0]):
            k = int(lp_count[b])
            for g in range(hkv):
                page_of[layer, b, g, :k] = perm[cursor:cursor + k]
                cursor += k
    return page_of, num_pages


def realize(w: Workload) -> Realized:
    cls = draw_classes(w)
    win = np.where(cls == 1, 0, w.window).astype(np.int32)
    c, n = draw_seqs(w)
    total = (c.astype(np.int64) + n).astype(np.int32)
    page_of, num_pages = allocate_pages(w.layers, w.hkv, w.page, total, w.seed, w.slack)
    return Realized(w=w, cached_len=c, new_len=n, head_class=cls, window=win,
                    page_of=page_of, num_pages=num_pages)


def relabel_pages(page_of: np.ndarray, num_pages: int, seed: int) -> np.ndarray:
    """Same logical layout, different physical pages: apply a seeded
    permutation of the pool ids to every entry (-1 stays -1)."""
    perm = _rng(seed, 4).permutation(num_pages).astype(np.int32)
    out = page_of.copy()
    m = out >= 0
    out[m] = perm[out[m]]
    return out


def layer_tensors(w: Workload, r: Realized, layer: int, device="cpu", tag: int = 0):
    """bf16 N(0, 1) tensors for one layer.

    Returns dict with
      q        [sum n_b][hq][d]      query rows of the new tokens, sequence-major
      k_cached [sum c_b][hkv][d]     K of the cached positions 0 .. c_b-1
      v_cached [sum c_b][hkv][d]
      k_new    [sum n_b][hkv][d]     K of the new positions c_b .. c_b+n_b-1
      v_new    [sum n_b][hkv][d]
    """
    import torch
    gen = torch.Generator(device=device)

    def draw(kind, rows, heads):
        gen.manual_seed(int(np.random.SeedSequence([w.seed, 5, layer, kind, tag]).generate_state(1)[0]))
        return torch.randn((rows, heads, w.d), generator=gen, device=device, dtype=torch.bfloat16)

    n_rows = int(r.new_len.sum())
    c_rows = int(r.cached_len.sum())
    return {
        "q": draw(0, n_rows, w.hq),
        "k_new": draw(1, n_rows, w.hkv),
        "v_new": draw(2, n_rows, w.hkv),
        "k_cached": draw(3, c_rows, w.hkv),
        "v_cached": draw(4, c_rows, w.hkv),
    }


def prefix(x: np.ndarray) -> np.ndarray:
    """Exclusive prefix sum with a leading 0 (int32), used to address packed rows."""
    out = np.zeros(x.shape[0] + 1, dtype=np.int64)
    np.cumsum(x, out=out[1:])
    return out.astype(np.int32)
