"""The allocation-free prefill entry point (segkv_attn_prefill_noalloc: the
split-KV workspace comes from the library's own device scratch) against
segkv_attn_prefill with a caller-owned workspace: same tables, same inputs,
identical bits. Two calls in a row on one device, the second with a smaller
workspace, so the second runs on scratch the first left behind."""

import ctypes

import pytest
import torch

import head_segmented_paged_amd as H
from head_segmented_paged_amd import segkv as S
from tests.common import adhoc
from workloads import layer_tensors, realize


class FakeDev:
    """Stand-in device pointer; never dereferenced by the host-side paths tested here."""

    def __init__(self, p):
        self.p = p

    def data_ptr(self):
        return self.p


def test_noalloc_rejects_oversized_workspace():
    """Tables whose partial results exceed the scratch are refused before
    anything is enqueued (host-side check, no device touched)."""
    w = adhoc(hq=8, hkv=2, d=128, page=64, window=0, classes=(1, 1), seqs=((0, 300),), seed=1)
    r = realize(w)
    ctx = H.segkv_create(FakeDev(1 << 20), FakeDev(1 << 21), w.hq, w.hkv, w.d, w.page, num_pages=r.num_pages)
    host = H.segkv_build_head_tables(ctx, r.cached_len, r.new_len, r.head_class[0], r.window[0], r.page_of[0])
    per_part = S.part_bytes(host["unit_rows"], host["unit_heads"], w.d)
    parts = S.NOALLOC_SCRATCH_BYTES // per_part + 1
    st = S.segkv_dev_tables(1 << 22, 1 << 23, 1 << 24, 1, 1, 1, host["total_q_rows"], host["unit_rows"],
                            host["unit_heads"], 1 << 25, 1, parts)
    rc = S._lib.segkv_attn_prefill_noalloc(ctx.handle, ctypes.byref(st), 1 << 26, 1 << 27, S.SEGKV_DTYPE_F32,
                                           None, 0.0, None)
    assert rc == S.SEGKV_ERR_CAPACITY
    assert "scratch" in H.segkv_last_error()
    st.num_parts = S.NOALLOC_SCRATCH_BYTES // per_part + 1
    st.unit_rows = 7    # a shape no kernel runs: refused as for segkv_attn_prefill
    rc = S._lib.segkv_attn_prefill_noalloc(ctx.handle, ctypes.byref(st), 1 << 26, 1 << 27, S.SEGKV_DTYPE_F32,
                                           None, 0.0, None)
    assert rc == S.SEGKV_ERR_INVALID_ARG


# larger workspace first, then smaller: (hq, hkv, d, page, window, classes, seqs, longest run in tiles).
# The first has more 256-pair units than CUs: its work queues sit in the scratch too.
CASES = [
    (8, 2, 128, 64, 1500, (1, 0), ((1000, 8300),), 64),
    (8, 2, 128, 64, 0, (1, 1), ((3000, 300),), 4),
    (4, 1, 128, 64, 500, (1,), ((900, 160),), 5),
]


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point():
    from tests.gpu_helpers import GpuLayer, say
    sizes = []
    for i, (hq, hkv, d, page, window, classes, seqs, run) in enumerate(CASES):
        say(f"[noalloc] case {i}: hq {hq} hkv {hkv} d {d} page {page} window {window} seqs {seqs} run {run}")
        w = adhoc(hq=hq, hkv=hkv, d=d, page=page, window=window, classes=classes, seqs=seqs, seed=31 + i)
        r = realize(w)
        gl = GpuLayer(w, r, 0, layer_tensors(w, r, 0), max_unit_tiles=run)
        gl.write()
        host = gl.tables()
        assert host["num_parts"] > 0 and host["num_merges"] > 0
        sizes.append(host["workspace_bytes"])
        rows = int(r.new_len.sum())
        q = gl.t["q"]
        for dt in (torch.float32, torch.bfloat16):
            o_ref = torch.full((rows, w.hq, w.d), float("nan"), dtype=dt, device="cuda")
            o_na = torch.full_like(o_ref, float("nan"))
            lse_ref = torch.full((w.hq, rows), float("nan"), dtype=torch.float32, device="cuda")
            lse_na = torch.full_like(lse_ref, float("nan"))
            H.segkv_attn_prefill(gl.ctx, gl.dev, q, o_ref, lse_ref)
            H.segkv_attn_prefill_noalloc(gl.ctx, gl.dev, q, o_na, lse_na)
            torch.cuda.synchronize()
            assert torch.isfinite(o_ref.float()).all()
            assert torch.equal(o_na, o_ref), f"case {i} {dt}: output differs"
            assert torch.equal(lse_na, lse_ref), f"case {i} {dt}: lse differs"
    assert sizes[2] < sizes[1] < sizes[0]
