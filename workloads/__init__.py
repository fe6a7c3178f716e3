"""Seeded synthetic prefill workloads (shapes, class tables, block tables, bf16 inputs)."""
from .configs import (ALL, BY_NAME, Workload, TINY, MISTRAL_8K, LLAMA70B_32K, STACK64_128K,  # noqa: F401
                      VARLEN_CHUNKED, DECODE_32K)
from .gen import Realized, realize, layer_tensors, relabel_pages, allocate_pages, prefix  # noqa: F401
