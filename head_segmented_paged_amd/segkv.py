"""Python binding of libsegkv (argument marshalling only).

Every function forwards to the C entry point of the same name declared in
include/segkv.h. Torch tensors are used only as device memory and for the
current HIP stream; all computation runs in the library's kernels. There is
no fallback: if libsegkv.so is missing, importing this module raises.
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsegkv.so")

SEGKV_OK = 0
SEGKV_ERR_INVALID_ARG = -1
SEGKV_ERR_OUT_OF_RANGE = -2
SEGKV_ERR_CAPACITY = -3
SEGKV_ERR_HIP = -4
SEGKV_ERR_UNSUPPORTED = -5
SEGKV_DTYPE_F32 = 0
SEGKV_DTYPE_BF16 = 1
NOALLOC_SCRATCH_BYTES = 64 << 20   # SEGKV_NOALLOC_SCRATCH_BYTES
SEG_FIELDS = 8
UNIT_FIELDS = 12
MERGE_FIELDS = 8


QUEUE_BYTES = 256                   # SEGKV_QUEUE_BYTES


def part_bytes(unit_rows, unit_heads, head_dim):
    """Workspace bytes per split-KV partial result (SEGKV_PART_BYTES)."""
    return 4 * unit_rows * unit_heads * (head_dim + 2)


def workspace_bytes(num_parts, unit_rows, unit_heads, head_dim):
    """Workspace segkv_attn_prefill needs (SEGKV_WORKSPACE_BYTES): the partial
    results, then for units of 256 pairs the persistent kernel's work queues."""
    queue = QUEUE_BYTES if unit_rows * unit_heads == 256 else 0
    return num_parts * part_bytes(unit_rows, unit_heads, head_dim) + queue
SEG_FIELD_NAMES = ("q_row0", "n_q", "q_pos0", "kv_head", "window", "k_pos0", "k_len", "page_off")

_P = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class segkv_config(ctypes.Structure):
    _fields_ = [("num_q_heads", _i32), ("num_kv_heads", _i32), ("head_dim", _i32), ("page_size", _i32),
                ("num_pages", _i64), ("k_pool", _P), ("v_pool", _P)]


class segkv_table_inputs(ctypes.Structure):
    _fields_ = [("num_seqs", _i32), ("max_lp", _i32), ("cached_len", _P), ("new_len", _P),
                ("head_class", _P), ("window", _P), ("page_of", _P), ("max_unit_tiles", _i32)]


class segkv_tables(ctypes.Structure):
    _fields_ = [("seg_cap", _i32), ("seq_cap", _i32), ("page_cap", _i64), ("unit_cap", _i32),
                ("num_segments", _i32), ("num_units", _i32), ("num_page_entries", _i64), ("total_pairs", _i64),
                ("total_q_rows", _i32), ("unit_rows", _i32), ("unit_heads", _i32),
                ("seg_desc", _P), ("cu_seqlens_q", _P), ("cu_seqlens_k", _P), ("cu_pages", _P),
                ("page_list", _P), ("pairs", _P), ("work", _P),
                ("merge_cap", _i32), ("num_merges", _i32), ("num_parts", _i32), ("workspace_bytes", _i64),
                ("merge", _P), ("retain_lp", _P)]


class segkv_dev_tables(ctypes.Structure):
    _fields_ = [("seg_desc", _P), ("page_list", _P), ("work", _P), ("num_segments", _i32), ("num_units", _i32),
                ("num_page_entries", _i64), ("total_q_rows", _i32), ("unit_rows", _i32), ("unit_heads", _i32),
                ("merge", _P), ("num_merges", _i32), ("num_parts", _i32)]


class SegKVError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"segkv error {code}: {message}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python head_segmented_paged_amd/build.py`")
    # torch brings its own HIP runtime under the same soname (libamdhip64.so.7).
    # Load it first, so the library binds to that one copy: with two runtimes
    # in one process the library's would see no device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "segkv_create": ([ctypes.POINTER(segkv_config), ctypes.POINTER(_P)], ctypes.c_int),
        "segkv_destroy": ([_P], None),
        "segkv_write_pages": ([_P, _P, _P, _i64, _P, _P, _P, _i32, _i32, _i32, _P], ctypes.c_int),
        "segkv_build_head_tables": ([_P, ctypes.POINTER(segkv_table_inputs), ctypes.POINTER(segkv_tables)],
                                    ctypes.c_int),
        "segkv_attn_prefill": ([_P, ctypes.POINTER(segkv_dev_tables), _P, _P, _i32, _P, ctypes.c_float, _P, _i64,
                                _P], ctypes.c_int),
        "segkv_attn_prefill_noalloc": ([_P, ctypes.POINTER(segkv_dev_tables), _P, _P, _i32, _P, ctypes.c_float, _P],
                                       ctypes.c_int),
        "segkv_gather_pages": ([_P, _P, _i64, _P, _P, _P], ctypes.c_int),
        "segkv_rope_realign": ([_P, _P, _i64, ctypes.c_float, _P], ctypes.c_int),
        "segkv_attn_mass": ([_P, ctypes.POINTER(segkv_dev_tables), _P, _P, ctypes.c_float, _P, _P], ctypes.c_int),
        "segkv_select_tokens": ([_P, _P, _P, _P, _P, _i32, _i64, _P, _P], ctypes.c_int),
        "segkv_sparse_ffn": ([_P, _P, _i64, _i32, _i32, _P, _i64, _P, _P, _P, _P, _i64, _P], ctypes.c_int),
        "segkv_last_error": ([], ctypes.c_char_p),
        "segkv_version": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()
EXPORTED = ("segkv_create", "segkv_destroy", "segkv_write_pages", "segkv_build_head_tables",
            "segkv_attn_prefill", "segkv_attn_prefill_noalloc", "segkv_attn_mass", "segkv_select_tokens", "segkv_sparse_ffn", "segkv_gather_pages",
            "segkv_rope_realign", "segkv_last_error", "segkv_version")


def segkv_last_error() -> str:
    return _lib.segkv_last_error().decode()


def segkv_version() -> str:
    return _lib.segkv_version().decode()


def _check(rc):
    if rc != SEGKV_OK:
        raise SegKVError(rc, segkv_last_error())


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        return x.ctypes.data_as(ctypes.c_void_p)
    return ctypes.c_void_p(x.data_ptr())


def _tensor(name, t, dtype=None, shape=None, device=None, min_numel=None):
    """Argument check before a C call (the C side cannot see tensor sizes, and
    a wrong size or stride there means out-of-bounds device accesses): a
    contiguous torch tensor on the expected device, with the given dtype and
    shape (None entries of shape are not checked). Checks only, no arithmetic."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None:
        if t.dim() != len(shape) or any(e is not None and int(a) != int(e) for a, e in zip(t.shape, shape)):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)} (None: any)")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs at least {min_numel}")
    return t


def _ctx_device(ctx):
    """Device of the context's pools (None for stand-in pools without one)."""
    import torch
    return ctx.k_pool.device if isinstance(ctx.k_pool, torch.Tensor) else None


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


class Context:
    """Owns a segkv_ctx and keeps the pool tensors alive."""

    def __init__(self, handle, cfg, k_pool, v_pool):
        self.handle = handle
        self.cfg = cfg
        self.k_pool = k_pool
        self.v_pool = v_pool

    @property
    def G(self):
        return self.cfg.num_q_heads // self.cfg.num_kv_heads

    def __del__(self):
        # at interpreter exit the module's globals may already be gone; the
        # process's end then releases the context
        if getattr(self, "handle", None) and _lib is not None:
            _lib.segkv_destroy(self.handle)
            self.handle = None


def segkv_create(k_pool, v_pool, num_q_heads, num_kv_heads, head_dim, page_size, num_pages=None):
    """k_pool: bf16 [num_pages][page_size][head_dim]; v_pool: bf16 [num_pages][head_dim][page_size]."""
    import torch
    if num_pages is None:
        num_pages = k_pool.shape[0] if k_pool is not None else 0
    if isinstance(k_pool, torch.Tensor) or isinstance(v_pool, torch.Tensor):
        _tensor("k_pool", k_pool, torch.bfloat16, (num_pages, page_size, head_dim))
        _tensor("v_pool", v_pool, torch.bfloat16, (num_pages, head_dim, page_size), device=k_pool.device)
    cfg = segkv_config(num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                       _ptr(k_pool) if k_pool is not None else None,
                       _ptr(v_pool) if v_pool is not None else None)
    h = ctypes.c_void_p()
    _check(_lib.segkv_create(ctypes.byref(cfg), ctypes.byref(h)))
    return Context(h, cfg, k_pool, v_pool)


def segkv_destroy(ctx: Context):
    if ctx.handle:
        _lib.segkv_destroy(ctx.handle)
        ctx.handle = None


def segkv_write_pages(ctx, k_new, v_new, cu_rows, pos0, page_of, max_rows_per_seq, stream=None):
    """k_new/v_new bf16 [rows][hkv][D]; cu_rows [S+1], pos0 [S], page_of [S][hkv][max_lp]: device int32."""
    import torch
    num_seqs = pos0.shape[0]
    max_lp = page_of.shape[-1]
    dev, cfg = _ctx_device(ctx), ctx.cfg
    _tensor("k_new", k_new, torch.bfloat16, (None, cfg.num_kv_heads, cfg.head_dim), dev)
    _tensor("v_new", v_new, torch.bfloat16, tuple(k_new.shape), dev)
    _tensor("cu_rows", cu_rows, torch.int32, (num_seqs + 1,), dev)
    _tensor("pos0", pos0, torch.int32, (num_seqs,), dev)
    _tensor("page_of", page_of, torch.int32, (num_seqs, cfg.num_kv_heads, max_lp), dev)
    _check(_lib.segkv_write_pages(ctx.handle, _ptr(k_new), _ptr(v_new), k_new.shape[0], _ptr(cu_rows),
                                  _ptr(pos0), _ptr(page_of), num_seqs, max_lp, int(max_rows_per_seq),
                                  _stream(stream)))


def segkv_build_head_tables(ctx, cached_len, new_len, head_class, window, page_of, max_unit_tiles=0):
    """Host arrays in, dict of host numpy arrays out (see segkv_tables in the header).
    max_unit_tiles: split-KV policy (0 automatic, > 0 longest run in tiles, < 0 never)."""
    c = np.ascontiguousarray(cached_len, dtype=np.int32)
    n = np.ascontiguousarray(new_len, dtype=np.int32)
    cls = np.ascontiguousarray(head_class, dtype=np.int8)
    win = np.ascontiguousarray(window, dtype=np.int32)
    po = np.ascontiguousarray(page_of, dtype=np.int32)
    inp = segkv_table_inputs(c.shape[0], po.shape[-1], _ptr(c), _ptr(n), _ptr(cls), _ptr(win), _ptr(po),
                             int(max_unit_tiles))
    out = segkv_tables()
    rc = _lib.segkv_build_head_tables(ctx.handle, ctypes.byref(inp), ctypes.byref(out))
    if rc not in (SEGKV_OK, SEGKV_ERR_CAPACITY):
        _check(rc)
    S = out.num_segments
    bufs = {
        "seg_desc": np.zeros((S, SEG_FIELDS), np.int32),
        "cu_seqlens_q": np.zeros(c.shape[0] + 1, np.int32),
        "cu_seqlens_k": np.zeros(S + 1, np.int32),
        "cu_pages": np.zeros(S + 1, np.int32),
        "page_list": np.zeros(max(out.num_page_entries, 1), np.int32),
        "pairs": np.zeros(S, np.int64),
        "work": np.zeros((max(out.num_units, 1), UNIT_FIELDS), np.int32),
        "merge": np.zeros((max(out.num_merges, 1), MERGE_FIELDS), np.int32),
        "retain_lp": np.zeros(S, np.int32),
    }
    out2 = segkv_tables(S, c.shape[0], bufs["page_list"].shape[0], bufs["work"].shape[0])
    out2.merge_cap = bufs["merge"].shape[0]
    for k, v in bufs.items():
        setattr(out2, k, _ptr(v))
    _check(_lib.segkv_build_head_tables(ctx.handle, ctypes.byref(inp), ctypes.byref(out2)))
    res = dict(bufs)
    res["page_list"] = res["page_list"][:out2.num_page_entries]
    res["work"] = res["work"][:out2.num_units]
    res["merge"] = res["merge"][:out2.num_merges]
    for i, name in enumerate(SEG_FIELD_NAMES):
        res[name] = res["seg_desc"][:, i].copy()
    for k in ("num_segments", "num_units", "num_page_entries", "total_pairs", "total_q_rows",
              "unit_rows", "unit_heads", "num_merges", "num_parts", "workspace_bytes"):
        res[k] = int(getattr(out2, k))
    return res


class DevTables:
    """Device copies of one layer's tables plus the struct handed to the kernel."""

    def __init__(self, host, device):
        import torch
        self.seg_desc = torch.from_numpy(np.ascontiguousarray(host["seg_desc"])).to(device)
        pl = host["page_list"] if host["page_list"].size else np.zeros(1, np.int32)
        self.page_list = torch.from_numpy(np.ascontiguousarray(pl)).to(device)
        wk = host["work"] if host["work"].size else np.zeros((1, UNIT_FIELDS), np.int32)
        self.work = torch.from_numpy(np.ascontiguousarray(wk)).to(device)
        mg = host["merge"] if host["merge"].size else np.zeros((1, MERGE_FIELDS), np.int32)
        self.merge = torch.from_numpy(np.ascontiguousarray(mg)).to(device)
        self.workspace_bytes = host["workspace_bytes"]
        self.host = host
        self.struct = segkv_dev_tables(_ptr(self.seg_desc), _ptr(self.page_list), _ptr(self.work),
                                       host["num_segments"], host["num_units"], host["num_page_entries"],
                                       host["total_q_rows"], host["unit_rows"], host["unit_heads"],
                                       _ptr(self.merge), host["num_merges"], host["num_parts"])


def upload_tables(host, device="cuda"):
    return DevTables(host, device)


def _attn_args(ctx, dev_tables, q, o, lse):
    """q bf16 [rows][hq][D], o [rows][hq][D] (dtype checked by the caller),
    lse fp32 [hq][rows] or None; rows = the tables' total_q_rows."""
    import torch
    rows, cfg, dev = int(dev_tables.struct.total_q_rows), ctx.cfg, _ctx_device(ctx)
    _tensor("q", q, torch.bfloat16, (rows, cfg.num_q_heads, cfg.head_dim), dev)
    if o is not None:
        _tensor("o", o, None, (rows, cfg.num_q_heads, cfg.head_dim), q.device)
    if lse is not None:
        _tensor("lse", lse, torch.float32, (cfg.num_q_heads, rows), q.device)


def segkv_attn_prefill(ctx, dev_tables, q, o, lse=None, softmax_scale=0.0, stream=None, workspace=None):
    """q bf16 [rows][hq][D]; o fp32 or bf16 [rows][hq][D]; lse fp32 [hq][rows] or None.
    workspace: device buffer of at least the tables' workspace_bytes (split-KV
    partial results, the work queues); when None and the tables need one, a
    torch buffer is allocated for the call."""
    import torch
    if o.dtype == torch.float32:
        dt = SEGKV_DTYPE_F32
    elif o.dtype == torch.bfloat16:
        dt = SEGKV_DTYPE_BF16
    else:
        raise TypeError("o must be float32 or bfloat16")
    _attn_args(ctx, dev_tables, q, o, lse)
    st = dev_tables.struct
    need = workspace_bytes(int(st.num_parts), int(st.unit_rows), int(st.unit_heads), ctx.cfg.head_dim)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _tensor("workspace", workspace, device=q.device, min_numel=need // workspace.element_size())
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.segkv_attn_prefill(ctx.handle, ctypes.byref(dev_tables.struct), _ptr(q), _ptr(o), dt,
                                   _ptr(lse), float(softmax_scale), _ptr(workspace), ws_bytes, _stream(stream)))


def segkv_attn_prefill_noalloc(ctx, dev_tables, q, o, lse=None, softmax_scale=0.0, stream=None):
    """segkv_attn_prefill with the split-KV workspace taken from the library's
    own device scratch (NOALLOC_SCRATCH_BYTES per GPU): no allocation by the
    call; calls that overlap on one GPU race."""
    import torch
    if o.dtype == torch.float32:
        dt = SEGKV_DTYPE_F32
    elif o.dtype == torch.bfloat16:
        dt = SEGKV_DTYPE_BF16
    else:
        raise TypeError("o must be float32 or bfloat16")
    _attn_args(ctx, dev_tables, q, o, lse)
    _check(_lib.segkv_attn_prefill_noalloc(ctx.handle, ctypes.byref(dev_tables.struct), _ptr(q), _ptr(o), dt,
                                           _ptr(lse), float(softmax_scale), _stream(stream)))


def segkv_attn_mass(ctx, dev_tables, q, lse, mass, softmax_scale=0.0, stream=None):
    """Attention mass of the new tokens: mass fp32 [rows], lse fp32 [hq][rows] from segkv_attn_prefill."""
    import torch
    rows = int(dev_tables.struct.total_q_rows)
    _attn_args(ctx, dev_tables, q, None, lse)
    _tensor("lse", lse, torch.float32, (ctx.cfg.num_q_heads, rows), q.device)
    _tensor("mass", mass, torch.float32, (rows,), q.device)
    _check(_lib.segkv_attn_mass(ctx.handle, ctypes.byref(dev_tables.struct), _ptr(q), _ptr(lse),
                                float(softmax_scale), _ptr(mass), _stream(stream)))


def segkv_select_tokens(ctx, mass, cu_rows, keep, cu_keep, rows_out, stream=None):
    """Top-keep[b] rows of each sequence by mass (ties to the lower row), ascending, into rows_out."""
    import torch
    S = keep.shape[0]
    _tensor("mass", mass, torch.float32, (None,))
    _tensor("cu_rows", cu_rows, torch.int32, (S + 1,), mass.device)
    _tensor("keep", keep, torch.int32, (S,), mass.device)
    _tensor("cu_keep", cu_keep, torch.int32, (S + 1,), mass.device)
    _tensor("rows_out", rows_out, torch.int32, (None,), mass.device)
    _check(_lib.segkv_select_tokens(ctx.handle, _ptr(mass), _ptr(cu_rows), _ptr(keep), _ptr(cu_keep),
                                    keep.shape[0], mass.shape[0], _ptr(rows_out), _stream(stream)))


def segkv_sparse_ffn(ctx, x, sel_rows, w_gate, w_up, w_down, h=None, stream=None):
    """x bf16 [rows][d_model] updated in place for the rows in sel_rows (int32 device);
    weights bf16 [d_ff][d_model] (gate, up) and [d_model][d_ff] (down); h: bf16 workspace or None."""
    import torch
    n_sel, d_ff, d_model = sel_rows.shape[0], w_gate.shape[0], x.shape[1]
    _tensor("x", x, torch.bfloat16, (None, d_model))
    _tensor("sel_rows", sel_rows, torch.int32, (n_sel,), x.device)
    _tensor("w_gate", w_gate, torch.bfloat16, (d_ff, d_model), x.device)
    _tensor("w_up", w_up, torch.bfloat16, (d_ff, d_model), x.device)
    _tensor("w_down", w_down, torch.bfloat16, (d_model, d_ff), x.device)
    if h is None:
        h = torch.empty((max(n_sel, 1), d_ff), dtype=torch.bfloat16, device=x.device)
    _tensor("h", h, torch.bfloat16, (None, d_ff), x.device)
    _check(_lib.segkv_sparse_ffn(ctx.handle, _ptr(x), x.shape[0], d_model, d_ff, _ptr(sel_rows), n_sel,
                                 _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(h), h.numel() * h.element_size(),
                                 _stream(stream)))


def segkv_rope_realign(ctx, entries, rope_base=10000.0, stream=None):
    """entries: device int32 [n][4] = (page, slot0, nslots, delta); rotates those K slots in place."""
    import torch
    _tensor("entries", entries, torch.int32, (None, 4), _ctx_device(ctx))
    _check(_lib.segkv_rope_realign(ctx.handle, _ptr(entries), entries.shape[0], float(rope_base), _stream(stream)))


def segkv_gather_pages(ctx, page_ids, k_out, v_out, stream=None):
    """page_ids device int32 [n]; k_out/v_out bf16 [n][P][D]."""
    import torch
    n, dev, cfg = page_ids.shape[0], _ctx_device(ctx), ctx.cfg
    _tensor("page_ids", page_ids, torch.int32, (n,), dev)
    _tensor("k_out", k_out, torch.bfloat16, (n, cfg.page_size, cfg.head_dim), dev)
    _tensor("v_out", v_out, torch.bfloat16, (n, cfg.page_size, cfg.head_dim), dev)
    _check(_lib.segkv_gather_pages(ctx.handle, _ptr(page_ids), page_ids.shape[0], _ptr(k_out), _ptr(v_out),
                                   _stream(stream)))
