#!/usr/bin/env python3
"""SegPaged prefill benchmark on one MI355X.

One step is one pass of the whole hot path over the 64-layer 128K stack
(32 query / 8 KV heads, head dim 128, page 64, window 2048; each (layer, KV
head) global with probability 0.13, layers 0-7 all local):
  * per layer, the host builds the head-class page tables and work list
    (segkv_build_head_tables) and uploads them asynchronously;
  * the layer's new K/V rows are written into their pages (segkv_write_pages);
  * the fused varlen attention runs over every head's visible keys
    (segkv_attn_prefill, bf16 output).
Layers run one after another on one stream, as a real prefill would. All
inputs (Q, K, V for every layer, the block tables, the pools) are resident in
HBM before the timed region.

The headline value is useful TFLOP/s: 4 * head_dim FLOPs per visible
(query, key) pair per query head, over the step time. The roofline object
reports the attention kernel alone against the bf16 MFMA peak, timed with HIP
events on the launch stream. A bounded sample of the fp64 CPU oracle runs
beside it on the host cores.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
# Sources whose change invalidates the committed HBM counter figures: the
# attention kernel and the work-list order that decides its cache reuse.
TRAFFIC_SOURCES = ("head_segmented_paged_amd/csrc/segkv_attn.hip", "head_segmented_paged_amd/csrc/segkv_tile_asm.inc",
                   "head_segmented_paged_amd/csrc/segkv_tables.cpp")
METRIC = "SegPagedAttention prefill TFLOP/s + ms/layer at 32K/128K; % bf16 MFMA peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class LayerTables:
    """One layer's tables: rebuilt on the host each step, uploaded through
    pinned buffers on the launch stream."""

    def __init__(self, H, S, torch, ctx, r, layer, device):
        self.H, self.torch, self.ctx = H, torch, ctx
        self.args = (r.cached_len, r.new_len, r.head_class[layer], r.window[layer], r.page_of[layer])
        host = H.segkv_build_head_tables(ctx, *self.args)
        self.keys = ("seg_desc", "page_list", "work", "merge")
        shape = {k: host[k].shape if host[k].size else (1, host[k].shape[-1]) for k in self.keys}
        self.pin = {k: torch.empty(shape[k], dtype=torch.int32, pin_memory=True) for k in self.keys}
        self.dev = {k: torch.empty(shape[k], dtype=torch.int32, device=device) for k in self.keys}
        self.pairs = host["total_pairs"]
        # split-KV partial results (none on the 128K stack and the 32K layer)
        self.workspace = torch.empty(max(host["workspace_bytes"], 1), dtype=torch.uint8, device=device)
        self.struct = S.segkv_dev_tables(
            self.dev["seg_desc"].data_ptr(), self.dev["page_list"].data_ptr(), self.dev["work"].data_ptr(),
            host["num_segments"], host["num_units"], host["num_page_entries"], host["total_q_rows"],
            host["unit_rows"], host["unit_heads"], self.dev["merge"].data_ptr(), host["num_merges"],
            host["num_parts"])
        self.free = torch.cuda.Event()
        self.free.record()

    def refresh(self):
        self.free.synchronize()            # the previous upload from the pinned buffers is done
        host = self.H.segkv_build_head_tables(self.ctx, *self.args)
        for k in self.keys:
            if host[k].size:
                self.pin[k].numpy()[...] = host[k]
            self.dev[k].copy_(self.pin[k], non_blocking=True)
        self.free.record()
        self.pairs = host["total_pairs"]


class Resident:
    """A workload with every layer's inputs resident on the GPU."""

    def __init__(self, w, device="cuda", o_dtype="bf16"):
        import torch
        import head_segmented_paged_amd as H
        from head_segmented_paged_amd import segkv as S
        from workloads import layer_tensors, prefix, realize
        self.torch, self.H, self.w = torch, H, w
        r = self.r = realize(w)
        t0 = time.perf_counter()
        self.k_pool = torch.zeros((r.num_pages, w.page, w.d), dtype=torch.bfloat16, device=device)
        self.v_pool = torch.zeros((r.num_pages, w.d, w.page), dtype=torch.bfloat16, device=device)
        self.ctx = H.segkv_create(self.k_pool, self.v_pool, w.hq, w.hkv, w.d, w.page)
        self.page_of = torch.from_numpy(np.ascontiguousarray(r.page_of)).to(device)
        self.cu_new = torch.from_numpy(prefix(r.new_len)).to(device)
        self.pos0 = torch.from_numpy(np.ascontiguousarray(r.cached_len, dtype=np.int32)).to(device)
        self.layers = []
        for layer in range(w.layers):
            t = layer_tensors(w, r, layer, device=device)
            if int(r.cached_len.sum()) > 0:      # the reused cache exists before the request
                cu_c = torch.from_numpy(prefix(r.cached_len)).to(device)
                zeros = torch.zeros_like(self.pos0)
                H.segkv_write_pages(self.ctx, t["k_cached"], t["v_cached"], cu_c, zeros, self.page_of[layer],
                                    int(r.cached_len.max()))
            self.layers.append({"q": t["q"], "k_new": t["k_new"], "v_new": t["v_new"]})
            del t
        rows = int(r.new_len.sum())
        odt = torch.bfloat16 if o_dtype == "bf16" else torch.float32
        self.o = torch.empty((rows, w.hq, w.d), dtype=odt, device=device)
        self.tables = [LayerTables(H, S, torch, self.ctx, r, layer, device) for layer in range(w.layers)]
        torch.cuda.synchronize()
        self.setup_s = time.perf_counter() - t0
        self.pairs_per_step = sum(int(lt.pairs) for lt in self.tables)
        self.flops_per_step = 4.0 * w.d * self.pairs_per_step

    def step(self, events=None):
        H, r = self.H, self.r
        max_new = int(r.new_len.max())
        for layer, lt in enumerate(self.tables):
            lt.refresh()
            x = self.layers[layer]
            if events is not None:
                events[layer][0].record()
            H.segkv_write_pages(self.ctx, x["k_new"], x["v_new"], self.cu_new, self.pos0, self.page_of[layer],
                                max_new)
            if events is not None:
                events[layer][1].record()
            H.segkv_attn_prefill(self.ctx, lt, x["q"], self.o, workspace=lt.workspace)
            if events is not None:
                events[layer][2].record()

    def timed(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in self.tables]
               for _ in range(steps)]
        t0 = time.perf_counter()
        for s in range(steps):
            self.step(evs[s])
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        attn = np.array([[e[1].elapsed_time(e[2]) for e in st] for st in evs])    # ms [steps][layers]
        write = np.array([[e[0].elapsed_time(e[1]) for e in st] for st in evs])
        return wall, attn, write


def measured_traffic(workload):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, or None when it was taken on another kernel or work-list source
    or another workload."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "attn_prefill_hbm_traffic.json")
    try:
        rec = json.load(open(path))
        sha = hashlib.sha256()
        for f in TRAFFIC_SOURCES:
            sha.update(open(os.path.join(ROOT, f), "rb").read())
        sha = sha.hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != sha or workload not in rec.get("workloads", {}):
        return None
    return float(rec["workloads"][workload]["bytes_per_launch"])


def algorithmic_bytes(w, r, o_bytes=2):
    """Bytes one attention launch must move, averaged over the layers: every Q
    row once, every K/V row visible to some query of a (sequence, KV head)
    segment once, every O row once."""
    rows = int(r.new_len.sum())
    qo = rows * w.hq * w.d * (2 + o_bytes)
    kv = 0
    for layer in range(w.layers):
        for b in range(r.num_seqs):
            c, T = int(r.cached_len[b]), int(r.cached_len[b] + r.new_len[b])
            for g in range(w.hkv):
                win = int(r.window[layer][g])
                lo = 0 if win == 0 else max(0, c - win + 1)
                kv += (T - lo) * w.d * 2 * 2
    return qo + kv / w.layers


def write_path(w, r, ms_per_step):
    """segkv_write_pages over the step: every new K and V row read once from
    the caller's [rows][hkv][D] buffers and written once into its page, per
    layer; GB/s against the HBM peak."""
    rows = int(r.new_len.sum())
    nbytes = 2 * 2 * rows * w.hkv * w.d * 2 * w.layers    # (read + write) x (K, V) x bf16
    gbs = nbytes / (ms_per_step / 1e3) / 1e9
    return {"bytes_per_step": nbytes, "ms_per_step": ms_per_step, "GB/s": gbs, "frac_hbm_peak": gbs / PEAK_HBM_GBS}


def cpu_baseline(res, target_s=18.0):
    """The fp64 oracle, as it stands, on a bounded sample of one layer's queries."""
    from oracle import paged as opaged
    from oracle import tables as otables
    torch, w, r = res.torch, res.w, res.r
    layer = int(np.argmax(r.head_class.sum(axis=1)))
    from workloads import layer_tensors
    t = layer_tensors(w, r, layer, device="cuda")
    bits = {k: opaged.bf16_bits(v) for k, v in t.items()}
    del t
    tab = otables.build_tables(r.cached_len, r.new_len, r.head_class[layer], r.window[layer], r.page_of[layer],
                               w.hq, w.hkv, w.page, r.num_pages)
    kp, vp = opaged.empty_pools(r.num_pages, w.page, w.d)
    opaged.scatter_pages(kp, vp, r.page_of[layer], r.cached_len, r.new_len, bits["k_cached"], bits["v_cached"],
                         bits["k_new"], bits["v_new"])
    rng = np.random.Generator(np.random.PCG64(2024))
    G = w.hq // w.hkv

    def sample(per_head):
        qs = []
        for b in range(r.num_seqs):
            n = int(r.new_len[b])
            for h in range(w.hq):
                tt = rng.integers(0, n, size=per_head)
                qs.append(np.stack([np.full(per_head, b), np.full(per_head, h), tt], 1))
        q = np.concatenate(qs).astype(np.int32)
        c = r.cached_len[q[:, 0]].astype(np.int64)
        win = r.window[layer][q[:, 1] // G].astype(np.int64)
        i = c + q[:, 2]
        cnt = np.where(win == 0, i + 1, np.minimum(i + 1, np.maximum(win, 1)))
        return q, int(cnt.sum())

    q, pairs = sample(4)
    t0 = time.perf_counter()
    opaged.attention(kp, vp, bits["q"], tab, q)
    dt = time.perf_counter() - t0
    per_head = int(max(4, min(4096, 4 * target_s / max(dt, 1e-3))))
    q, pairs = sample(per_head)
    cores = opaged.threads()
    t0 = time.perf_counter()
    opaged.attention(kp, vp, bits["q"], tab, q)
    dt = time.perf_counter() - t0
    # one thread, on a sample about 1/cores as large (a few seconds)
    q1, pairs1 = sample(max(1, per_head // max(cores, 1)))
    opaged.set_threads(1)
    try:
        t0 = time.perf_counter()
        opaged.attention(kp, vp, bits["q"], tab, q1)
        dt1 = time.perf_counter() - t0
    finally:
        opaged.set_threads(cores)
    del kp, vp
    return {
        "value": 4.0 * w.d * pairs / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{len(q)} queries ({per_head} uniform rows per query head, all {w.hq} heads) of layer {layer} "
                   f"of {w.name}; {pairs} visible pairs in {dt:.1f} s; fp64"),
        "cpu_model": cpu_model(),
        "host_threads": os.cpu_count(),
        "ns_per_pair": dt / pairs * 1e9,
        "single_thread_ns_per_pair": dt1 / pairs1 * 1e9,
        "single_thread_sample": f"{len(q1)} queries, {pairs1} visible pairs in {dt1:.1f} s on 1 thread",
        "extrapolated_step_s": dt / pairs * res.pairs_per_step,
    }


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or the platform string."""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def ffn_bench(torch, steps, warmup, tokens=8192, keep=2048, d_model=4096, d_ff=14336):
    """The gathered SwiGLU FFN of `keep` chosen tokens out of `tokens` (a
    Mistral-7B-sized block, random weights), timed with HIP events; the same
    kernels over every token give the dense FFN time for comparison."""
    import head_segmented_paged_amd as H
    g = torch.Generator(device="cuda").manual_seed(7)
    x = torch.randn((tokens, d_model), device="cuda", dtype=torch.bfloat16, generator=g)
    w = [(torch.randn(shape, device="cuda", dtype=torch.float32, generator=g) / shape[1] ** 0.5).to(torch.bfloat16)
         for shape in ((d_ff, d_model), (d_ff, d_model), (d_model, d_ff))]
    ctx = H.segkv_create(torch.zeros((1, 64, 128), dtype=torch.bfloat16, device="cuda"),
                         torch.zeros((1, 128, 64), dtype=torch.bfloat16, device="cuda"), 32, 8, 128, 64)
    rng = np.random.Generator(np.random.PCG64(5))
    sel = torch.from_numpy(np.sort(rng.choice(tokens, keep, replace=False)).astype(np.int32)).cuda()
    dense = torch.arange(tokens, dtype=torch.int32, device="cuda")
    h = torch.empty((tokens, d_ff), dtype=torch.bfloat16, device="cuda")

    def timeit(rows):
        for _ in range(warmup):
            H.segkv_sparse_ffn(ctx, x, rows, *w, h=h)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(steps):
            H.segkv_sparse_ffn(ctx, x, rows, *w, h=h)
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / steps

    ms = timeit(sel)
    ms_dense = timeit(dense)
    flops = 3 * 2.0 * keep * d_model * d_ff
    tf = flops / (ms / 1e3) / 1e12
    return {"metric": "sparse FFN of the chosen tokens (gathered SwiGLU, bf16 MFMA)", "value": tf,
            "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": ms,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"sparse_ffn_{keep}of{tokens}_dm{d_model}_dff{d_ff}", "tokens": tokens,
                       "chosen": keep, "d_model": d_model, "d_ff": d_ff},
            "dense_ms_all_tokens": ms_dense,
            "dense_tflops_all_tokens": 3 * 2.0 * tokens * d_model * d_ff / (ms_dense / 1e3) / 1e12,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / PEAK_BF16_TFLOPS, "traffic": None}}


def rope_bench(torch, n_pages, steps, warmup, P=64, D=128):
    """RoPE re-alignment of n_pages whole K pages (each turned by its own
    delta), timed with HIP events on the launch stream. Bytes = every K page
    read and written once."""
    import head_segmented_paged_amd as H
    k = torch.randn((n_pages, P, D), device="cuda", dtype=torch.bfloat16)
    v = torch.zeros((n_pages, D, P), device="cuda", dtype=torch.bfloat16)
    ctx = H.segkv_create(k, v, 32, 8, D, P, num_pages=n_pages)
    rng = np.random.Generator(np.random.PCG64(11))
    ent = np.stack([np.arange(n_pages), np.zeros(n_pages), np.full(n_pages, P),
                    rng.integers(-65536, 65536, n_pages)], 1).astype(np.int32)
    ent = torch.from_numpy(ent).cuda()
    for _ in range(warmup):
        H.segkv_rope_realign(ctx, ent)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(steps):
        H.segkv_rope_realign(ctx, ent)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    gbs = 2.0 * n_pages * P * D * 2 / (ms / 1e3) / 1e9
    return {"metric": "RoPE re-alignment of reused K pages", "value": gbs, "unit": "GB/s", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"rope_realign_{n_pages}pages_p{P}_d{D}", "pages": n_pages},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "traffic": None}}


def run_secondary(name, steps=5, warmup=2):
    from workloads import BY_NAME
    res = Resident(BY_NAME[name])
    wall, attn, write = res.timed(steps, warmup)
    a = float(np.median(attn.sum(axis=1)))
    out = {
        "workload": name,
        "ms_per_layer": a,
        "tflops": res.flops_per_step / (a / 1e3) / 1e12,
        "step_ms": wall * 1e3,
        "write_ms": float(np.median(write.sum(axis=1))),
    }
    out["pct_bf16_peak"] = 100.0 * out["tflops"] / PEAK_BF16_TFLOPS
    del res
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="stack64_l131072")
    ap.add_argument("--o-dtype", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (HBM counter calibration)")
    ap.add_argument("--sparse-ffn", action="store_true",
                    help="only time the sparse FFN of 2048 chosen of 8192 tokens (d_model 4096, d_ff 14336)")
    ap.add_argument("--rope-pages", type=int, default=0, metavar="N",
                    help="only time the RoPE re-alignment of N reused K pages (P 64, D 128), in GB/s")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    from workloads import BY_NAME
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return
    if args.sparse_ffn:
        print(json.dumps(ffn_bench(torch, args.steps, args.warmup)), flush=True)
        return
    if args.rope_pages:
        print(json.dumps(rope_bench(torch, args.rope_pages, args.steps, args.warmup)), flush=True)
        return
    w = BY_NAME[args.workload]
    log(f"[bench] setting up {w.name} ({w.layers} layers)")
    res = Resident(w, o_dtype=args.o_dtype)
    log(f"[bench] setup {res.setup_s:.1f} s; running {args.warmup} warmup + {args.steps} timed steps")
    wall, attn, write = res.timed(args.steps, args.warmup)
    attn_step = attn.sum(axis=1)                      # ms per step, attention launches only
    write_step = write.sum(axis=1)
    achieved = res.flops_per_step / (float(np.mean(attn_step)) / 1e3) / 1e12
    algo_bytes = algorithmic_bytes(w, res.r, 2 if args.o_dtype == "bf16" else 4)
    # A decode step (a few new rows per sequence) moves far more bytes than it
    # computes: its roofline is HBM bandwidth, not the matrix cores.
    decode = int(res.r.new_len.max()) <= 8
    if decode:
        roof = {"bound": "hbm", "achieved": algo_bytes * w.layers / (float(np.mean(attn_step)) / 1e3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(w.name)
    value = res.flops_per_step / wall / 1e12
    r = res.r
    globals_per_layer = r.head_class.sum(axis=1).tolist()
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "layers": w.layers, "seq_len": int(r.cached_len[0] + r.new_len[0]),
            "num_seqs": r.num_seqs, "q_heads": w.hq, "kv_heads": w.hkv, "head_dim": w.d, "page_size": w.page,
            "window": w.window, "global_kv_heads": int(sum(globals_per_layer)),
            "kv_heads_total": w.layers * w.hkv, "o_dtype": args.o_dtype,
        },
        "ms_per_layer": float(np.mean(attn_step)) / w.layers,
        "ms_per_layer_step": wall * 1e3 / w.layers,
        "attn_ms_total": float(np.mean(attn_step)),
        "write_ms_total": float(np.mean(write_step)),
        "write_path": write_path(w, res.r, float(np.mean(write_step))),
        "pct_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "visible_pairs_per_step": res.pairs_per_step,
        "useful_flops_per_step": res.flops_per_step,
        "roofline": roof,
        "algorithmic_bytes_per_launch": algo_bytes,
        "globals_per_layer": globals_per_layer,
        # mean attention time of the layers with 0, 1, 2, ... global KV heads
        "ms_per_layer_by_globals": {
            str(g): float(attn.mean(axis=0)[np.asarray(globals_per_layer) == g].mean())
            for g in sorted(set(globals_per_layer))},
    }
    if not args.no_secondary and w.name == "stack64_l131072":
        del res
        torch.cuda.empty_cache()
        log("[bench] secondary: llama70b_like_l32768")
        line["at_32k"] = run_secondary("llama70b_like_l32768")
        res = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle sample)")
        if res is None:
            res = Resident(w, o_dtype=args.o_dtype) if w.layers == 1 else _light(w)
        line["cpu_baseline"] = cpu_baseline(res)
    print(json.dumps(line), flush=True)


class _Light:
    pass


def _light(w):
    """Metadata-only stand-in for the CPU baseline (no GPU buffers)."""
    import torch
    from workloads import realize
    x = _Light()
    x.torch, x.w, x.r = torch, w, realize(w)
    from oracle import tables as otables
    x.pairs_per_step = 0
    for layer in range(w.layers):
        t = otables.build_tables(x.r.cached_len, x.r.new_len, x.r.head_class[layer], x.r.window[layer],
                                 x.r.page_of[layer], w.hq, w.hkv, w.page, x.r.num_pages)
        x.pairs_per_step += int(t["pairs"].sum())
    return x


if __name__ == "__main__":
    main()
