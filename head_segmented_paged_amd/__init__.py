"""Head-segmented paged KV cache + fused varlen prefill attention for MI355X (gfx950).

The compute lives in libsegkv.so (HIP kernels + host C++, C ABI in
include/segkv.h); this package is its Python binding.
"""
from .segkv import *  # noqa: F401,F403
from .segkv import (Context, DevTables, SegKVError, segkv_attn_mass, segkv_attn_prefill,  # noqa: F401
                    segkv_attn_prefill_noalloc,
                    segkv_build_head_tables,
                    segkv_create, segkv_destroy, segkv_gather_pages, segkv_last_error, segkv_rope_realign,
                    segkv_select_tokens, segkv_sparse_ffn,
                    segkv_version, segkv_write_pages, upload_tables)
