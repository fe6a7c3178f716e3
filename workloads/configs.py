"""Synthetic prefill workloads for head-segmented paged attention.

Each workload fixes the model shape (query heads, KV heads, head dim), the page
size, the sequences (cached length c_b and new length n_b per sequence), the
local window and the rule that labels each (layer, KV head) global or local.
The shapes follow the RedKnot summary page ("SegPaged Attention" and
"Head-Class Sparsification" sections): global heads are a small minority
(about 12-15 %), local heads reuse a sliding window, and shallow layers are
kept conservative (all local). Values are bf16 draws from N(0, 1); no dataset
or trained weight is involved.

This module holds only data. It computes nothing of the method itself.
"""

from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    hq: int                  # query heads
    hkv: int                 # KV heads
    d: int                   # head dim
    page: int                # tokens per page
    window: int              # local window W (tokens, including the query itself)
    # class rule:
    #   ("fixed", table)         explicit [layers][hkv] table, 1 = global
    #   ("count", k)             exactly k global KV heads per layer, positions from the seed
    #   ("bernoulli", p, n0)     each (layer, kv head) global with probability p; layers < n0 all local
    class_rule: Tuple
    # sequences:
    #   ("fixed", ((c, n), ...))              explicit cached / new lengths
    #   ("uniform_cached", nseq, lo, hi, n)   c_b integer-uniform in [lo, hi], n_b = n
    seq_rule: Tuple
    seed: int
    slack: float = 1.25      # pool capacity / pages needed (free pages exist to poison)
    note: str = ""


TINY = Workload(
    name="tiny_gqa2_l512",
    layers=1, hq=4, hkv=2, d=64, page=16, window=64,
    class_rule=("fixed", ((1, 0),)),
    seq_rule=("fixed", ((0, 512),)),
    seed=1001,
    note="1 layer, 4 q / 2 kv heads, D 64, L 512; kv0 global, kv1 local W 64; P 16",
)

MISTRAL_8K = Workload(
    name="mistral7b_like_l8192",
    layers=1, hq=32, hkv=8, d=128, page=64, window=1024,
    class_rule=("count", 1),
    seq_rule=("fixed", ((0, 8192),)),
    seed=1002,
    note="1 layer, 32 q / 8 kv, D 128, L 8192; 1 of 8 kv heads global, W 1024; P 64",
)

LLAMA70B_32K = Workload(
    name="llama70b_like_l32768",
    layers=1, hq=64, hkv=8, d=128, page=64, window=2048,
    class_rule=("count", 1),   # 15 % of 8 KV heads rounds to 1
    seq_rule=("fixed", ((0, 32768),)),
    seed=1003,
    note="1 layer, 64 q / 8 kv, D 128, L 32768; 1 of 8 kv heads global, W 2048; P 64",
)

STACK64_128K = Workload(
    name="stack64_l131072",
    layers=64, hq=32, hkv=8, d=128, page=64, window=2048,
    class_rule=("bernoulli", 0.13, 8),
    seq_rule=("fixed", ((0, 131072),)),
    seed=1004,
    note="64 layers, 32 q / 8 kv, D 128, L 131072; (layer, kv) global w.p. 0.13, "
         "layers 0-7 all local; W 2048; P 64",
)

VARLEN_CHUNKED = Workload(
    name="varlen16_chunk2048",
    layers=1, hq=32, hkv=8, d=128, page=64, window=1024,
    class_rule=("count", 1),
    seq_rule=("uniform_cached", 16, 2048, 32768, 2048),
    seed=1005,
    note="16 sequences, cached length U[2048, 32768], 2048 new query tokens each; "
         "32 q / 8 kv, D 128, 1 of 8 kv heads global, W 1024; P 64; one shared pool",
)

DECODE_32K = Workload(
    name="decode32_l32768",
    layers=1, hq=64, hkv=8, d=128, page=64, window=2048,
    class_rule=("count", 1),
    seq_rule=("fixed", tuple((32767, 1) for _ in range(32))),
    seed=1006,
    note="one decode step of 32 concurrent sequences at 32K: 32767 cached tokens and 1 new token each; "
         "64 q / 8 kv, D 128, 1 of 8 kv heads global, W 2048; P 64",
)

ALL = (TINY, MISTRAL_8K, LLAMA70B_32K, STACK64_128K, VARLEN_CHUNKED, DECODE_32K)
BY_NAME = {w.name: w for w in ALL}
