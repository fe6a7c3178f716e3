"""Oracle side of the paged KV pool and its attention call (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module. It shares no code with the library under test.

  * build()            compiles attn_fp64.c with the host C compiler (gcc, OpenMP).
  * scatter_pages()    the oracle's own paged write: every logical position of
                       every (sequence, KV head) is stored at slot pos % P of
                       the physical page page_of[b, g, pos // P] (block-table
                       mapping of the KV-cache management page, section 3.1;
                       per-head pages of the RedKnot summary page, "SegPaged
                       Attention"). Positions whose page id is -1 are skipped.
  * attention()        runs the fp64 oracle over a list of (b, h, t) queries.

Pool layout (shared storage contract, implemented here independently):
K pool uint16(bf16) [num_pages][P][D]; V pool uint16(bf16) [num_pages][D][P].
"""

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_fp64.c")
_LIB = os.path.join(_HERE, "liboracle_attn.so")


def build(src=_SRC, out=_LIB, extra=()):
    """Compile the C oracle. Plain -O2 with OpenMP; no target-specific flags,
    so the result runs on any x86-64 host."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", *extra, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib_cache = {}


def load(path=_LIB):
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path):
        build(out=path)
    lib = ctypes.CDLL(path)
    fn = lib.oracle_attn_fp64
    P = ctypes.c_void_p
    fn.argtypes = [P, P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                   P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_int32,
                   P, P, P, P, P, P, P, P, ctypes.c_int64,
                   P, ctypes.c_int64, ctypes.c_double, P, P]
    fn.restype = ctypes.c_int
    fm = lib.oracle_mass_fp64
    fm.argtypes = [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                   P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                   P, P, P, P, P, P, P, P, ctypes.c_int64,
                   P, ctypes.c_int64, ctypes.c_double, P]
    fm.restype = ctypes.c_int
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = None
    _lib_cache[path] = lib
    return lib


def threads(lib_path=_LIB):
    """OpenMP threads the oracle runs on."""
    return int(load(lib_path).oracle_threads())


def set_threads(n, lib_path=_LIB):
    """Threads of the oracle's parallel loop from now on (timing only)."""
    load(lib_path).oracle_set_threads(int(n))


def bf16_bits(x) -> np.ndarray:
    """uint16 view of a bf16 torch tensor (copied to host), or of uint16 numpy data."""
    if isinstance(x, np.ndarray):
        assert x.dtype == np.uint16
        return np.ascontiguousarray(x)
    import torch
    return x.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def empty_pools(num_pages, P, D):
    """Zero-initialised host pools. np.zeros maps untouched pages lazily, so a
    large pool costs memory only for the pages actually written."""
    return (np.zeros((num_pages, P, D), dtype=np.uint16),
            np.zeros((num_pages, D, P), dtype=np.uint16))


def scatter_pages(k_pool, v_pool, page_of_layer, cached_len, new_len,
                  k_cached, v_cached, k_new, v_new):
    """Write one layer's logical K/V rows into the host pools.

    page_of_layer  int [S][hkv][max_lp]
    k_cached/v_cached  uint16 [sum c_b][hkv][D]  positions 0..c_b-1 of each sequence
    k_new/v_new        uint16 [sum n_b][hkv][D]  positions c_b..c_b+n_b-1
    """
    P = k_pool.shape[1]
    nseq = len(cached_len)
    hkv = page_of_layer.shape[1]
    c_off = 0
    n_off = 0
    for b in range(nseq):
        c = int(cached_len[b])
        n = int(new_len[b])
        pos = np.arange(c + n, dtype=np.int64)
        for g in range(hkv):
            krows = np.concatenate([k_cached[c_off:c_off + c, g, :], k_new[n_off:n_off + n, g, :]])
            vrows = np.concatenate([v_cached[c_off:c_off + c, g, :], v_new[n_off:n_off + n, g, :]])
            pages = page_of_layer[b, g, pos // P].astype(np.int64)
            keep = pages >= 0
            p_k, s_k = pages[keep], (pos % P)[keep]
            k_pool[p_k, s_k, :] = krows[keep]
            v_pool[p_k, :, s_k] = vrows[keep]
        c_off += c
        n_off += n


def all_queries(tables, hq):
    """Every (b, h, t) of a layer, sequence-major, then head, then row."""
    G = tables["G"]
    hkv = tables["hkv"]
    out = []
    nseq = len(tables["cu_seqlens_q"]) - 1
    for b in range(nseq):
        n = int(tables["n_q"][b * hkv])
        for h in range(hq):
            t = np.arange(n, dtype=np.int32)
            out.append(np.stack([np.full(n, b, np.int32), np.full(n, h, np.int32), t], axis=1))
    del G
    return np.concatenate(out).astype(np.int32) if out else np.zeros((0, 3), np.int32)


def attention(k_pool, v_pool, q_bits, tables, queries, scale=None, lib_path=_LIB):
    """fp64 oracle attention for the given (b, h, t) queries.

    q_bits uint16 [sum n_b][hq][D]. Returns (o [nq][D] float64, lse [nq] float64).
    """
    lib = load(lib_path)
    num_pages, P, D = k_pool.shape
    hq, hkv = tables["hq"], tables["hkv"]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    queries = np.ascontiguousarray(queries, dtype=np.int32)
    nq = queries.shape[0]
    o = np.zeros((nq, D), dtype=np.float64)
    lse = np.zeros(nq, dtype=np.float64)
    arrs = {k: np.ascontiguousarray(tables[k], dtype=np.int32)
            for k in ("q_row0", "n_q", "q_pos0", "kv_head", "window", "k_pos0", "cu_pages", "page_list")}
    q_bits = np.ascontiguousarray(q_bits)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    rc = lib.oracle_attn_fp64(
        ptr(k_pool), ptr(v_pool), num_pages, P, D,
        ptr(q_bits), q_bits.shape[0], hq, hkv,
        len(arrs["q_row0"]),
        ptr(arrs["q_row0"]), ptr(arrs["n_q"]), ptr(arrs["q_pos0"]), ptr(arrs["kv_head"]),
        ptr(arrs["window"]), ptr(arrs["k_pos0"]), ptr(arrs["cu_pages"]),
        ptr(arrs["page_list"]), len(arrs["page_list"]),
        ptr(queries), nq, float(scale), ptr(o), ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_attn_fp64 failed with status {rc}")
    return o, lse


def attention_mass(k_pool, q_bits, tables, queries, scale=None, lib_path=_LIB):
    """fp64 attention mass of the new tokens (oracle_mass_fp64): float64 [sum n_b],
    summed over the given (b, h, t) queries (normally all of them)."""
    lib = load(lib_path)
    num_pages, P, D = k_pool.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    queries = np.ascontiguousarray(queries, dtype=np.int32)
    q_bits = np.ascontiguousarray(q_bits)
    mass = np.zeros(q_bits.shape[0], dtype=np.float64)
    arrs = {k: np.ascontiguousarray(tables[k], dtype=np.int32)
            for k in ("q_row0", "n_q", "q_pos0", "kv_head", "window", "k_pos0", "cu_pages", "page_list")}
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    rc = lib.oracle_mass_fp64(
        ptr(k_pool), num_pages, P, D, ptr(q_bits), q_bits.shape[0], tables["hq"], tables["hkv"],
        len(arrs["q_row0"]), ptr(arrs["q_row0"]), ptr(arrs["n_q"]), ptr(arrs["q_pos0"]), ptr(arrs["kv_head"]),
        ptr(arrs["window"]), ptr(arrs["k_pos0"]), ptr(arrs["cu_pages"]), ptr(arrs["page_list"]),
        len(arrs["page_list"]), ptr(queries), queries.shape[0], float(scale), ptr(mass))
    if rc != 0:
        raise ValueError(f"oracle_mass_fp64 failed with status {rc}")
    return mass
