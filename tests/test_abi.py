"""C-ABI boundary checks that need no GPU: the library loads, exports every
entry point the header declares, and rejects bad arguments with the
documented codes before anything would be enqueued."""

import ctypes
import os
import re

import numpy as np
import pytest

import head_segmented_paged_amd as H
from head_segmented_paged_amd import segkv as S
from tests.common import adhoc
from workloads import TINY, realize

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "segkv.h")


class FakeDev:
    """Stand-in device pointer; never dereferenced by the host-side paths tested here."""

    def __init__(self, p):
        self.p = p

    def data_ptr(self):
        return self.p


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|void|char)\s*\*?\s*(segkv_\w+)\s*\(", text, re.M)))


def test_header_declarations_are_exported():
    names = declared_functions()
    assert len(names) >= 8
    lib = ctypes.CDLL(S.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(S.EXPORTED)


def test_version():
    assert "gfx950" in H.segkv_version()


def _ctx(hq=4, hkv=2, d=64, p=16, pages=100):
    return H.segkv_create(FakeDev(1 << 20), FakeDev(1 << 21), hq, hkv, d, p, num_pages=pages)


@pytest.mark.parametrize("args,code", [
    ((5, 2, 64, 16, 100), S.SEGKV_ERR_INVALID_ARG),
    ((4, 0, 64, 16, 100), S.SEGKV_ERR_INVALID_ARG),
    ((4, 2, 96, 16, 100), S.SEGKV_ERR_UNSUPPORTED),
    ((4, 2, 64, 24, 100), S.SEGKV_ERR_UNSUPPORTED),
    ((4, 2, 64, 8, 100), S.SEGKV_ERR_UNSUPPORTED),
    ((4, 2, 64, 16, 0), S.SEGKV_ERR_INVALID_ARG),
])
def test_create_rejects(args, code):
    hq, hkv, d, p, pages = args
    with pytest.raises(S.SegKVError) as e:
        H.segkv_create(FakeDev(1), FakeDev(2), hq, hkv, d, p, num_pages=pages)
    assert e.value.code == code


def test_create_rejects_null_pool():
    with pytest.raises(S.SegKVError) as e:
        H.segkv_create(None, FakeDev(2), 4, 2, 64, 16, num_pages=10)
    assert e.value.code == S.SEGKV_ERR_INVALID_ARG


def test_tables_errors():
    r = realize(TINY)
    ctx = _ctx(pages=r.num_pages)
    args = (r.cached_len, r.new_len, r.head_class[0], r.window[0])
    po = r.page_of[0].copy()
    po[0, 1, 5] = -1
    with pytest.raises(S.SegKVError) as e:
        H.segkv_build_head_tables(ctx, *args, po)
    assert e.value.code == S.SEGKV_ERR_OUT_OF_RANGE
    po = r.page_of[0].copy()
    po[0, 0, 0] = r.num_pages
    with pytest.raises(S.SegKVError) as e:
        H.segkv_build_head_tables(ctx, *args, po)
    assert e.value.code == S.SEGKV_ERR_OUT_OF_RANGE
    with pytest.raises(S.SegKVError) as e:
        H.segkv_build_head_tables(ctx, r.cached_len, r.new_len, r.head_class[0], np.array([0, 0]), r.page_of[0])
    assert e.value.code == S.SEGKV_ERR_INVALID_ARG
    with pytest.raises(S.SegKVError) as e:
        H.segkv_build_head_tables(ctx, r.cached_len, np.array([0]), r.head_class[0], r.window[0], r.page_of[0])
    assert e.value.code == S.SEGKV_ERR_INVALID_ARG
    with pytest.raises(S.SegKVError) as e:
        H.segkv_build_head_tables(ctx, r.cached_len, r.new_len, r.head_class[0], r.window[0], r.page_of[0][:, :, :3])
    assert e.value.code == S.SEGKV_ERR_OUT_OF_RANGE


def test_tables_capacity_reports_sizes():
    r = realize(TINY)
    ctx = _ctx(pages=r.num_pages)
    c = np.ascontiguousarray(r.cached_len, np.int32)
    n = np.ascontiguousarray(r.new_len, np.int32)
    cls = np.ascontiguousarray(r.head_class[0], np.int8)
    win = np.ascontiguousarray(r.window[0], np.int32)
    po = np.ascontiguousarray(r.page_of[0], np.int32)
    inp = S.segkv_table_inputs(1, po.shape[-1], S._ptr(c), S._ptr(n), S._ptr(cls), S._ptr(win), S._ptr(po))
    out = S.segkv_tables()
    rc = S._lib.segkv_build_head_tables(ctx.handle, ctypes.byref(inp), ctypes.byref(out))
    assert rc == S.SEGKV_ERR_CAPACITY
    assert out.num_segments == 2 and out.num_page_entries == 64 and out.total_q_rows == 512
    assert out.total_pairs == 324_160


def test_attn_prefill_validates_before_launch():
    r = realize(TINY)
    ctx = _ctx(pages=r.num_pages)
    host = H.segkv_build_head_tables(ctx, r.cached_len, r.new_len, r.head_class[0], r.window[0], r.page_of[0])
    dt = S.segkv_dev_tables(1, 2, 3, host["num_segments"], host["num_units"], host["num_page_entries"],
                            host["total_q_rows"], host["unit_rows"] * 2, host["unit_heads"])
    rc = S._lib.segkv_attn_prefill(ctx.handle, ctypes.byref(dt), 4, 5, S.SEGKV_DTYPE_F32, None, 0.0, None, 0, None)
    assert rc == S.SEGKV_ERR_INVALID_ARG and "units" in H.segkv_last_error()
    dt.unit_rows = host["unit_rows"]
    rc = S._lib.segkv_attn_prefill(ctx.handle, ctypes.byref(dt), 4, 5, 7, None, 0.0, None, 0, None)
    assert rc == S.SEGKV_ERR_INVALID_ARG
    rc = S._lib.segkv_attn_prefill(ctx.handle, ctypes.byref(dt), None, 5, S.SEGKV_DTYPE_F32, None, 0.0, None, 0, None)
    assert rc == S.SEGKV_ERR_INVALID_ARG
    rc = S._lib.segkv_attn_prefill(None, ctypes.byref(dt), 4, 5, S.SEGKV_DTYPE_F32, None, 0.0, None, 0, None)
    assert rc == S.SEGKV_ERR_INVALID_ARG


def test_split_tables_need_a_workspace():
    w = adhoc(hq=4, hkv=1, d=128, page=64, window=64, classes=(1,), seqs=((0, 300),), seed=5)
    r = realize(w)
    ctx = _ctx(w.hq, w.hkv, w.d, w.page, r.num_pages)
    host = H.segkv_build_head_tables(ctx, r.cached_len, r.new_len, r.head_class[0], r.window[0], r.page_of[0],
                                     max_unit_tiles=2)
    assert host["num_parts"] > 0 and host["num_merges"] > 0
    pairs = host["unit_rows"] * host["unit_heads"]
    assert host["workspace_bytes"] == host["num_parts"] * 4 * pairs * (w.d + 2) + (256 if pairs == 256 else 0)
    dt = S.segkv_dev_tables(1, 2, 3, host["num_segments"], host["num_units"], host["num_page_entries"],
                            host["total_q_rows"], host["unit_rows"], host["unit_heads"], 9, host["num_merges"],
                            host["num_parts"])
    rc = S._lib.segkv_attn_prefill(ctx.handle, ctypes.byref(dt), 4, 5, S.SEGKV_DTYPE_F32, None, 0.0, None, 0, None)
    assert rc == S.SEGKV_ERR_CAPACITY and "workspace" in H.segkv_last_error()
    rc = S._lib.segkv_attn_prefill(ctx.handle, ctypes.byref(dt), 4, 5, S.SEGKV_DTYPE_F32, None, 0.0, 8,
                                   host["workspace_bytes"] - 1, None)
    assert rc == S.SEGKV_ERR_CAPACITY
    dt.merge = None
    rc = S._lib.segkv_attn_prefill(ctx.handle, ctypes.byref(dt), 4, 5, S.SEGKV_DTYPE_F32, None, 0.0, 8,
                                   host["workspace_bytes"], None)
    assert rc == S.SEGKV_ERR_INVALID_ARG and "merge" in H.segkv_last_error()
    # pages shorter than a tile: the builder never splits, hand-made split tables are refused
    ctx16 = _ctx(4, 1, 128, 16, 64)
    dt.unit_rows, dt.unit_heads = 32, 4          # the short-page kernel's unit: four waves, G = 4
    dt.merge = 9
    rc = S._lib.segkv_attn_prefill(ctx16.handle, ctypes.byref(dt), 4, 5, S.SEGKV_DTYPE_F32, None, 0.0, 8,
                                   host["workspace_bytes"], None)
    assert rc == S.SEGKV_ERR_UNSUPPORTED


def test_rope_realign_validates_before_launch():
    ctx = _ctx(d=128, p=64)
    rc = S._lib.segkv_rope_realign(ctx.handle, None, 3, 10000.0, None)
    assert rc == S.SEGKV_ERR_INVALID_ARG and "entries" in H.segkv_last_error()
    rc = S._lib.segkv_rope_realign(ctx.handle, 8, -1, 10000.0, None)
    assert rc == S.SEGKV_ERR_INVALID_ARG
    rc = S._lib.segkv_rope_realign(ctx.handle, 8, 3, 1.0, None)
    assert rc == S.SEGKV_ERR_INVALID_ARG and "rope_base" in H.segkv_last_error()
    assert S._lib.segkv_rope_realign(ctx.handle, None, 0, 10000.0, None) == S.SEGKV_OK   # nothing to do
    assert S._lib.segkv_rope_realign(None, 8, 3, 10000.0, None) == S.SEGKV_ERR_INVALID_ARG


def test_write_and_gather_validate_before_launch():
    ctx = _ctx()
    rc = S._lib.segkv_write_pages(ctx.handle, None, 2, 10, 3, 4, 5, 1, 4, 16, None)
    assert rc == S.SEGKV_ERR_INVALID_ARG
    rc = S._lib.segkv_write_pages(ctx.handle, 1, 2, 10, 3, 4, 5, 0, 4, 16, None)
    assert rc == S.SEGKV_ERR_INVALID_ARG
    rc = S._lib.segkv_write_pages(ctx.handle, 1, 2, 0, 3, 4, 5, 1, 4, 16, None)
    assert rc == S.SEGKV_OK                      # nothing to write: no launch
    rc = S._lib.segkv_gather_pages(ctx.handle, None, 3, 1, 2, None)
    assert rc == S.SEGKV_ERR_INVALID_ARG
    rc = S._lib.segkv_gather_pages(ctx.handle, 1, -1, 1, 2, None)
    assert rc == S.SEGKV_ERR_INVALID_ARG


def test_binding_checks_tensors_before_calling():
    """The binding refuses mis-shaped, mistyped or strided tensors before the
    C call (the library cannot see tensor sizes; a wrong one would mean
    out-of-bounds device accesses). CPU tensors: nothing reaches a device."""
    import torch
    hq, hkv, d, p, n = 4, 2, 64, 16, 10
    kp = torch.zeros((n, p, d), dtype=torch.bfloat16)
    vp = torch.zeros((n, d, p), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        H.segkv_create(kp, torch.zeros((n, p, d), dtype=torch.bfloat16), hq, hkv, d, p)   # V not transposed
    with pytest.raises(TypeError):
        H.segkv_create(kp.float(), vp, hq, hkv, d, p)
    with pytest.raises(ValueError):
        H.segkv_create(kp, vp.transpose(1, 2).contiguous().transpose(1, 2), hq, hkv, d, p)   # strided view
    ctx = H.segkv_create(kp, vp, hq, hkv, d, p)
    w = adhoc(hq=hq, hkv=hkv, d=d, page=p, window=8, classes=(1, 0), seqs=((0, 40),), seed=3)
    r = realize(w)
    host = H.segkv_build_head_tables(ctx, r.cached_len, r.new_len, r.head_class[0], r.window[0], r.page_of[0])
    st = S.segkv_dev_tables(1 << 20, 1 << 21, 1 << 22, host["num_segments"], host["num_units"],
                            host["num_page_entries"], host["total_q_rows"], host["unit_rows"], host["unit_heads"],
                            None, 0, 0)

    class Tables:
        struct = st
    rows = host["total_q_rows"]
    q = torch.zeros((rows, hq, d), dtype=torch.bfloat16)
    o = torch.zeros((rows, hq, d), dtype=torch.float32)
    for bad_q in (q[:-1], q.float(), q.transpose(0, 1).contiguous().transpose(0, 1), torch.zeros((rows, hq, 2 * d))):
        with pytest.raises((TypeError, ValueError)):
            H.segkv_attn_prefill(ctx, Tables, bad_q, o)
        with pytest.raises((TypeError, ValueError)):
            H.segkv_attn_prefill_noalloc(ctx, Tables, bad_q, o)
    with pytest.raises(ValueError):
        H.segkv_attn_prefill(ctx, Tables, q, o[:, :2])
    with pytest.raises(ValueError):
        H.segkv_attn_prefill(ctx, Tables, q, o, lse=torch.zeros((rows, hq), dtype=torch.float32))
    with pytest.raises(ValueError):
        H.segkv_write_pages(ctx, torch.zeros((5, hkv + 1, d), dtype=torch.bfloat16),
                            torch.zeros((5, hkv + 1, d), dtype=torch.bfloat16),
                            torch.zeros(2, dtype=torch.int32), torch.zeros(1, dtype=torch.int32),
                            torch.zeros((1, hkv, 4), dtype=torch.int32), 5)
    with pytest.raises(ValueError):
        H.segkv_rope_realign(ctx, torch.zeros((3, 3), dtype=torch.int32))


def test_binding_workspace_matches_builder():
    """The binding sizes the workspace it allocates with the builder's formula:
    the partial results, and for 256-pair units the persistent kernel's work
    queues (SEGKV_QUEUE_BYTES)."""
    for seqs, run in (((0, 300),), 2), (((0, 8192),), 0):
        w = adhoc(hq=8, hkv=2, d=128, page=64, window=0, classes=(1, 1), seqs=seqs, seed=3)
        r = realize(w)
        ctx = _ctx(w.hq, w.hkv, w.d, w.page, r.num_pages)
        host = H.segkv_build_head_tables(ctx, r.cached_len, r.new_len, r.head_class[0], r.window[0], r.page_of[0],
                                         max_unit_tiles=run)
        pairs = host["unit_rows"] * host["unit_heads"]
        assert S.workspace_bytes(host["num_parts"], host["unit_rows"], host["unit_heads"], w.d) == \
            host["workspace_bytes"]
        assert (host["workspace_bytes"] % S.part_bytes(host["unit_rows"], host["unit_heads"], w.d) ==
                (S.QUEUE_BYTES if pairs == 256 else 0))
