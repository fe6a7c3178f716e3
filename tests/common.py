"""Shared test helpers: build a layer's inputs, the oracle's tables and pools."""

from dataclasses import dataclass, field, replace

import numpy as np

from oracle import paged as opaged
from oracle import tables as otables
from workloads import Workload, layer_tensors, prefix, realize, relabel_pages


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclass
class Case:
    w: Workload
    layer: int
    cached_len: np.ndarray
    new_len: np.ndarray
    head_class: np.ndarray      # [hkv] of this layer
    window: np.ndarray          # [hkv]
    page_of: np.ndarray         # [S][hkv][max_lp] of this layer
    num_pages: int
    bits: dict                  # uint16 arrays: q, k_new, v_new, k_cached, v_cached
    tables: dict = None
    k_pool: np.ndarray = None
    v_pool: np.ndarray = None
    extra: dict = field(default_factory=dict)

    @property
    def scale(self):
        return 1.0 / np.sqrt(self.w.d)

    def dense_kv(self):
        """Per sequence dense logical K/V [c+n][hkv][D] as float64."""
        cu_c = prefix(self.cached_len)
        cu_n = prefix(self.new_len)
        ks, vs = [], []
        for b in range(len(self.cached_len)):
            kc = self.bits["k_cached"][cu_c[b]:cu_c[b + 1]]
            kn = self.bits["k_new"][cu_n[b]:cu_n[b + 1]]
            vc = self.bits["v_cached"][cu_c[b]:cu_c[b + 1]]
            vn = self.bits["v_new"][cu_n[b]:cu_n[b + 1]]
            ks.append(bits_to_f64(np.concatenate([kc, kn])))
            vs.append(bits_to_f64(np.concatenate([vc, vn])))
        return ks, vs


def adhoc(hq=4, hkv=2, d=16, page=16, window=8, classes=(1, 0), seqs=((0, 40),), seed=7, slack=1.25):
    return Workload(name="adhoc", layers=1, hq=hq, hkv=hkv, d=d, page=page, window=window,
                    class_rule=("fixed", (tuple(classes),)), seq_rule=("fixed", tuple(seqs)),
                    seed=seed, slack=slack)


def make_case(w: Workload, layer=0, relabel_seed=None, bits=None, build=True):
    """Realize workload w, draw layer tensors on the CPU (unless bits are given),
    and, with build=True, run the oracle's table builder and paged write."""
    r = realize(w)
    page_of = r.page_of
    if relabel_seed is not None:
        page_of = relabel_pages(page_of, r.num_pages, relabel_seed)
    if bits is None:
        t = layer_tensors(w, r, layer, device="cpu")
        bits = {k: opaged.bf16_bits(v) for k, v in t.items()}
    case = Case(w=w, layer=layer, cached_len=r.cached_len, new_len=r.new_len,
                head_class=r.head_class[layer], window=r.window[layer],
                page_of=page_of[layer], num_pages=r.num_pages, bits=bits)
    if build:
        build_oracle_state(case)
    return case


def build_oracle_state(case: Case):
    w = case.w
    case.tables = otables.build_tables(case.cached_len, case.new_len, case.head_class, case.window,
                                       case.page_of, w.hq, w.hkv, w.page, case.num_pages)
    case.k_pool, case.v_pool = opaged.empty_pools(case.num_pages, w.page, w.d)
    opaged.scatter_pages(case.k_pool, case.v_pool, case.page_of, case.cached_len, case.new_len,
                         case.bits["k_cached"], case.bits["v_cached"],
                         case.bits["k_new"], case.bits["v_new"])
    return case


def oracle_all(case: Case, lib_path=None):
    """Oracle output for every query of the layer, as [sum n][hq][D] and [sum n][hq]."""
    q = opaged.all_queries(case.tables, case.w.hq)
    kw = {} if lib_path is None else {"lib_path": lib_path}
    o, lse = opaged.attention(case.k_pool, case.v_pool, case.bits["q"], case.tables, q, **kw)
    return scatter_rows(case, q, o, lse)


def scatter_rows(case, queries, o, lse):
    """Place per-query results at [q_row0 + t][h]."""
    hkv = case.w.hkv
    rows = case.tables["q_row0"][queries[:, 0] * hkv] + queries[:, 2]
    O = np.full((int(case.new_len.sum()), case.w.hq, case.w.d), np.nan)
    L = np.full((int(case.new_len.sum()), case.w.hq), np.nan)
    O[rows, queries[:, 1]] = o
    L[rows, queries[:, 1]] = lse
    return O, L


def with_window(w: Workload, window: int) -> Workload:
    return replace(w, window=window)
