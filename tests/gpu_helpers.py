"""GPU-side drivers for the parity tests: run the library's write + table +
attention path on cuda:0 for one layer and hand back host results."""

import sys

import numpy as np
import torch

import head_segmented_paged_amd as H
from oracle import paged as opaged
from workloads import prefix


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def device_pools(num_pages, P, D, fill=0.0, device="cuda"):
    k = torch.full((num_pages, P, D), fill, dtype=torch.bfloat16, device=device)
    v = torch.full((num_pages, D, P), fill, dtype=torch.bfloat16, device=device)
    return k, v


class GpuLayer:
    """One layer of a realized workload on the GPU."""

    def __init__(self, w, r, layer, tensors, page_of=None, poison=False, device="cuda", pools=None,
                 max_unit_tiles=0):
        self.w, self.r, self.layer = w, r, layer
        self.max_unit_tiles = max_unit_tiles
        self.page_of = (r.page_of[layer] if page_of is None else page_of).astype(np.int32)
        if pools is None:
            pools = device_pools(r.num_pages, w.page, w.d, float("nan") if poison else 0.0, device)
        self.k_pool, self.v_pool = pools
        self.ctx = H.segkv_create(self.k_pool, self.v_pool, w.hq, w.hkv, w.d, w.page)
        self.t = {k: v.to(device) for k, v in tensors.items()}
        self.device = device

    def write(self, stream=None):
        r = self.r
        po = torch.from_numpy(np.ascontiguousarray(self.page_of)).to(self.device)
        zeros = torch.zeros(r.num_seqs, dtype=torch.int32, device=self.device)
        if int(r.cached_len.sum()) > 0:
            cu_c = torch.from_numpy(prefix(r.cached_len)).to(self.device)
            H.segkv_write_pages(self.ctx, self.t["k_cached"], self.t["v_cached"], cu_c, zeros, po,
                                int(r.cached_len.max()), stream)
        cu_n = torch.from_numpy(prefix(r.new_len)).to(self.device)
        pos0 = torch.from_numpy(np.ascontiguousarray(r.cached_len, dtype=np.int32)).to(self.device)
        H.segkv_write_pages(self.ctx, self.t["k_new"], self.t["v_new"], cu_n, pos0, po, int(r.new_len.max()), stream)

    def tables(self):
        r = self.r
        self.host = H.segkv_build_head_tables(self.ctx, r.cached_len, r.new_len, r.head_class[self.layer],
                                              r.window[self.layer], self.page_of, self.max_unit_tiles)
        self.dev = H.upload_tables(self.host, self.device)
        return self.host

    def attention(self, o_dtype=torch.float32, with_lse=True, stream=None):
        rows = int(self.r.new_len.sum())
        o = torch.empty((rows, self.w.hq, self.w.d), dtype=o_dtype, device=self.device)
        lse = torch.empty((self.w.hq, rows), dtype=torch.float32, device=self.device) if with_lse else None
        H.segkv_attn_prefill(self.ctx, self.dev, self.t["q"], o, lse, 0.0, stream)
        return o, lse

    def run(self, o_dtype=torch.float32):
        self.write()
        self.tables()
        o, lse = self.attention(o_dtype)
        torch.cuda.synchronize()
        return o, lse


def host_bits(t):
    return opaged.bf16_bits(t)


def sample_rows(n, c, W, P, rng, n_uniform=256, edge=64):
    """Row indices t (0 <= t < n) for sampled parity: the first and last rows,
    rows whose absolute position sits at the window edge and at page
    boundaries, plus seeded-uniform rows."""
    s = set(range(min(edge, n)))
    s.update(range(max(0, n - edge), n))
    for pos in list(range(W - 2, W + 2)) + [P - 1, P, 8 * P - 1, 8 * P, 8 * P + 1]:
        for t in (pos - c, pos):
            if 0 <= t < n:
                s.add(t)
    if n_uniform:
        s.update(int(x) for x in rng.integers(0, n, size=n_uniform))
    return np.array(sorted(s), dtype=np.int32)


def compare(gpu_o, gpu_lse, ora_o, ora_lse, queries, tables, hkv, max_abs=1e-2, mean_abs=1e-3, lse_abs=2e-3):
    """gpu_o [rows][hq][D], gpu_lse [hq][rows] (torch, any device) vs oracle per-query results."""
    rows = tables["q_row0"][queries[:, 0] * hkv] + queries[:, 2]
    heads = queries[:, 1]
    g = gpu_o.float().cpu().numpy()[rows, heads].astype(np.float64)
    err = np.abs(g - ora_o)
    stats = {"max_abs": float(err.max()), "mean_abs": float(err.mean()), "n": int(len(rows))}
    assert np.isfinite(g).all(), "non-finite GPU output"
    assert stats["max_abs"] <= max_abs, stats
    assert stats["mean_abs"] <= mean_abs, stats
    if gpu_lse is not None:
        gl = gpu_lse.cpu().numpy()[heads, rows].astype(np.float64)
        lerr = np.abs(gl - ora_lse)
        stats["lse_max_abs"] = float(lerr.max())
        assert stats["lse_max_abs"] <= lse_abs, stats
    return stats
