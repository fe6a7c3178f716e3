"""GPU parity of the attention mass of the new tokens (segkv_attn_mass)
against the fp64 oracle (oracle_mass_fp64), through the C ABI.

Bar: |mass - oracle| <= 4e-3 * oracle + 1e-5 per token. The kernel weighs
each score with the attention kernel's own LSE, which is within 2e-3 of the
exact one (the attention parity bar), so each weight is within about 2e-3
relative; a sum of positive weights keeps that relative error. The float
atomics make the summation order vary from run to run: results are checked
against the oracle, not against each other bit for bit."""

import numpy as np
import pytest
import torch

import head_segmented_paged_amd as H
from oracle import paged as opaged
from oracle import tables as otables
from tests.common import adhoc
from tests.gpu_helpers import GpuLayer, host_bits, say
from workloads import MISTRAL_8K, layer_tensors, realize

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]



def _one_page_ctx(hq, hkv, D=128, P=64):
    """A context for the token choice and the FFN, which read no pool: one-page pools."""
    k = torch.zeros((1, P, D), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((1, D, P), dtype=torch.bfloat16, device="cuda")
    return H.segkv_create(k, v, hq, hkv, D, P)

def run_mass(w, max_unit_tiles=0, unit_pairs=None):
    r = realize(w)
    say(f"[case] mass {w.name} hq {w.hq} hkv {w.hkv} D {w.d} P {w.page} "
        f"seqs {list(zip(r.cached_len.tolist(), r.new_len.tolist()))[:4]} run {max_unit_tiles}")
    t = layer_tensors(w, r, 0, device="cuda")
    gl = GpuLayer(w, r, 0, t, max_unit_tiles=max_unit_tiles)
    o, lse = gl.run()
    if unit_pairs is not None:
        assert gl.host["unit_rows"] * gl.host["unit_heads"] == unit_pairs
    mass = torch.empty(int(r.new_len.sum()), dtype=torch.float32, device="cuda")
    H.segkv_attn_mass(gl.ctx, gl.dev, t["q"], lse, mass)
    torch.cuda.synchronize()
    bits = {k: host_bits(v) for k, v in t.items()}
    tab = otables.build_tables(r.cached_len, r.new_len, r.head_class[0], r.window[0], r.page_of[0],
                               w.hq, w.hkv, w.page, r.num_pages)
    kp, vp = opaged.empty_pools(r.num_pages, w.page, w.d)
    opaged.scatter_pages(kp, vp, r.page_of[0], r.cached_len, r.new_len, bits["k_cached"], bits["v_cached"],
                         bits["k_new"], bits["v_new"])
    ref = opaged.attention_mass(kp, bits["q"], tab, opaged.all_queries(tab, w.hq))
    got = mass.cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    say(f"[ok] mass: max rel {np.max(err / np.maximum(ref, 1e-9)):.2e}, total {got.sum():.6g} vs {ref.sum():.6g}")
    assert np.all(err <= 4e-3 * ref + 1e-5)
    return got, ref


MASS = [
    # (hq, hkv, d, page, window, classes, seqs, longest run)
    (8, 2, 128, 64, 100, (0, 1), ((0, 200), (37, 301), (1000, 77)), 0),
    (16, 2, 64, 128, 300, (1, 0), ((250, 260), (0, 40)), 0),
    (6, 3, 128, 256, 40, (1, 0, 0), ((700, 45), (3, 250)), 0),
    (4, 4, 64, 64, 1, (1, 1, 0, 0), ((130, 70), (64, 64)), 2),
    (8, 2, 128, 64, 2000, (1, 0), ((0, 513),), 3),
]


@pytest.mark.parametrize("case", MASS, ids=lambda c: f"hq{c[0]}_kv{c[1]}_d{c[2]}_p{c[3]}_w{c[4]}_run{c[7]}")
def test_mass_all_tokens(case):
    hq, hkv, d, page, window, classes, seqs, run = case
    run_mass(adhoc(hq=hq, hkv=hkv, d=d, page=page, window=window, classes=classes, seqs=seqs, seed=hq * d + page),
             max_unit_tiles=run)


MASS_WIDE = [
    # long cached prefixes (mean visible keys per row >= 2048): eight-wave units
    (8, 1, 128, 64, 0, (1,), ((3000, 300),), 0),
    (4, 2, 64, 128, 3000, (1, 0), ((2500, 200), (4000, 77)), 4),
    (2, 2, 128, 256, 0, (1, 1), ((2100, 513),), 0),
]


@pytest.mark.parametrize("case", MASS_WIDE, ids=lambda c: f"hq{c[0]}_kv{c[1]}_d{c[2]}_p{c[3]}_run{c[7]}")
def test_mass_wide_units(case):
    hq, hkv, d, page, window, classes, seqs, run = case
    run_mass(adhoc(hq=hq, hkv=hkv, d=d, page=page, window=window, classes=classes, seqs=seqs, seed=hq + d + page),
             max_unit_tiles=run, unit_pairs=256)


def test_mass_8k():
    got, ref = run_mass(MISTRAL_8K)
    # no cached prefix: every query's weights sum to one over the new tokens
    assert abs(got.sum() - 32 * 8192) <= 1e-3 * 32 * 8192


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_select_tokens_matches_oracle(seed):
    from oracle.sparse_ffn import select_tokens
    rng = np.random.Generator(np.random.PCG64(100 + seed))
    n = np.array([1, 7, 1023, 1024, 1025, 5000, 70000, 333])
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    mass = (np.round(rng.random(cu[-1]) * 50) / 7).astype(np.float32)       # ties, and exact zeros
    mass[rng.random(cu[-1]) < 0.01] = np.nan
    mass[rng.random(cu[-1]) < 0.01] = -1.0
    keep = np.array([1, 0, 1000, 1024, 2000, 1, 17000, 333], dtype=np.int32)
    k = np.minimum(keep, n)
    cu_keep = np.concatenate([[0], np.cumsum(k)]).astype(np.int32)
    say(f"[case] select seed {seed}: {len(n)} sequences, {cu[-1]} rows")
    ctx = _one_page_ctx(8, 2)
    dev = {name: torch.from_numpy(a).cuda() for name, a in
           (("mass", mass), ("cu", cu), ("keep", keep), ("cu_keep", cu_keep))}
    out = torch.full((int(cu_keep[-1]),), -7, dtype=torch.int32, device="cuda")
    H.segkv_select_tokens(ctx, dev["mass"], dev["cu"], dev["keep"], dev["cu_keep"], out)
    torch.cuda.synchronize()
    expect = select_tokens(mass.astype(np.float64), cu, keep, cu_keep)
    assert np.array_equal(out.cpu().numpy(), expect)


def test_mass_then_select_8k():
    """End to end on the 8K layer: mass from the attention's LSE, then the
    top quarter of the tokens; the choice equals the oracle's on the same masses."""
    from oracle.sparse_ffn import select_tokens
    got, ref = run_mass(MISTRAL_8K)
    n = got.shape[0]
    ctx = _one_page_ctx(32, 8)
    m = torch.from_numpy(got.astype(np.float32)).cuda()
    cu = torch.tensor([0, n], dtype=torch.int32, device="cuda")
    keep = torch.tensor([n // 4], dtype=torch.int32, device="cuda")
    cu_keep = torch.tensor([0, n // 4], dtype=torch.int32, device="cuda")
    out = torch.empty(n // 4, dtype=torch.int32, device="cuda")
    H.segkv_select_tokens(ctx, m, cu, keep, cu_keep, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), select_tokens(got.astype(np.float32).astype(np.float64), [0, n], [n // 4]))


@pytest.mark.parametrize("dm,dff,rows,nsel", [(256, 512, 300, 77), (128, 384, 50, 50), (4096, 14336, 1024, 200)])
def test_sparse_ffn_matches_oracle(dm, dff, rows, nsel):
    """End to end against the oracle's whole step (oracle.sparse_ffn on the
    input x: its own h, its own residual; no kernel value reaches the oracle).
    h: |got - ref| <= one bf16 ulp of ref + 2^-20 x (the sum of the absolute
    terms that formed the value), at most 1 % of the values off at all (fp32
    sums over d_model terms are within ~1e-6 of the sum of absolute terms;
    where those cancel that bound holds, otherwise only values within that of
    a rounding midpoint round the other way).
    x, chosen rows: the kernel's h may be off by that h bound, which W_down
    carries into the row: |got - ref| <= one bf16 ulp of ref
    + sum_k |Wd[j,k]| (ulp(h_ref[k]) + 2^-20 h_terms[k]) + 2^-20 y_terms[j],
    y_terms = |x| + |h_ref| @ |Wd|^T.
    Every other row of x is unchanged bit for bit."""
    from oracle import sparse_ffn as osf
    say(f"[case] sparse ffn d_model {dm} d_ff {dff} rows {rows} chosen {nsel}")
    g = torch.Generator(device="cpu").manual_seed(dm + nsel)
    x = torch.randn((rows, dm), generator=g).to(torch.bfloat16)
    wg = (torch.randn((dff, dm), generator=g) / dm ** 0.5).to(torch.bfloat16)
    wu = (torch.randn((dff, dm), generator=g) / dm ** 0.5).to(torch.bfloat16)
    wd = (torch.randn((dm, dff), generator=g) / dff ** 0.5).to(torch.bfloat16)
    sel = np.sort(np.random.Generator(np.random.PCG64(nsel)).choice(rows, nsel, replace=False)).astype(np.int32)
    ctx = _one_page_ctx(8, 2)
    xd = x.cuda()
    h = torch.empty((nsel, dff), dtype=torch.bfloat16, device="cuda")
    H.segkv_sparse_ffn(ctx, xd, torch.from_numpy(sel).cuda(), wg.cuda(), wu.cuda(), wd.cuda(), h)
    torch.cuda.synchronize()
    b = lambda t: t.view(torch.int16).numpy().view(np.uint16)    # noqa: E731
    xb, hb = b(xd.cpu()), b(h.cpu())
    x0 = b(x)
    x_ref, h_ref = osf.sparse_ffn(x0, sel, b(wg), b(wu), b(wd))

    f = osf._bits_to_f64

    def ulp(bits):
        return np.ldexp(1.0, np.frexp(np.maximum(np.abs(f(bits)), 1e-30))[1] - 8)   # bf16 spacing at |value|

    def check(got, ref, bound, what, max_off=None):
        err = np.abs(f(got) - f(ref))
        off = err > 0
        say(f"[ok] {what}: {off.mean():.2e} of values off, worst error / bound {np.max(err / bound):.3f}")
        assert np.all(err <= bound)
        if max_off is not None:
            assert off.mean() <= max_off

    xs = f(x0[sel])
    g_, u_ = xs @ f(b(wg)).T, xs @ f(b(wu)).T
    ag, au = np.abs(xs) @ np.abs(f(b(wg))).T, np.abs(xs) @ np.abs(f(b(wu))).T
    h_terms = 1.1 * ag * np.abs(u_) + np.abs(osf.silu(g_)) * au
    h_bound = ulp(h_ref) * 1.0001 + 2.0 ** -20 * h_terms
    check(hb, h_ref, h_bound, "h", max_off=0.01)
    awd = np.abs(f(b(wd)))
    y_terms = np.abs(xs) + np.abs(f(h_ref)) @ awd.T
    x_bound = ulp(x_ref[sel]) * 1.0001 + h_bound @ awd.T + 2.0 ** -20 * y_terms
    check(xb[sel], x_ref[sel], x_bound, "x chosen rows")
    keep = np.ones(rows, bool)
    keep[sel] = False
    assert np.array_equal(xb[keep], x0[keep])
