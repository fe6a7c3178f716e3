// Randomised driver for the sanitizer build (address + undefined-behaviour
// sanitizers, host code only): the library's table builder and argument
// validation with the device launchers stubbed out, and the C oracle on small
// paged cases laid out by the builder's own tables.
//
//   fuzz_host <seed> <iterations>
//
// Inputs cover valid layers (global and local heads, windows of 1 and wider
// than the context, single-row and long chunks, every page size, every
// split-KV policy) and invalid ones (bad page ids, a max_lp too short, bad
// lengths and windows), the two-call capacity protocol (sizes first, then
// exact buffers; a buffer one short must be refused), and the attention
// entry points' host-side checks. Exit status 0 iff every call returned the
// code expected of it and every table invariant checked here held.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "segkv.h"

extern "C" int oracle_attn_fp64(const uint16_t *k_pool, const uint16_t *v_pool, int64_t num_pages, int32_t P,
                                int32_t D, const uint16_t *q, int64_t q_rows, int32_t hq, int32_t hkv,
                                int32_t num_segments, const int32_t *q_row0, const int32_t *n_q,
                                const int32_t *q_pos0, const int32_t *kv_head, const int32_t *window,
                                const int32_t *k_pos0, const int32_t *cu_pages, const int32_t *page_list,
                                int64_t page_list_len, const int32_t *queries, int64_t num_queries, double scale,
                                double *o, double *lse);

namespace {

std::mt19937_64 rng;
int64_t rnd(int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(rng); }
template <class T> T pick(std::initializer_list<T> v) { return *(v.begin() + rnd(0, static_cast<int64_t>(v.size()) - 1)); }

int failures = 0;
void expect(bool ok, const char *what, int it)
{
    if (!ok) {
        ++failures;
        std::fprintf(stderr, "iteration %d: %s (last error: %s)\n", it, what, segkv_last_error());
    }
}

struct Buffers {
    std::vector<int32_t> seg_desc, cu_q, cu_k, cu_pages, page_list, work, merge, retain;
    std::vector<int64_t> pairs;
    void bind(segkv_tables &t, int seg, int seq, int64_t pages, int units, int merges)
    {
        seg_desc.assign(static_cast<size_t>(seg) * SEGKV_SEG_FIELDS, -7);
        cu_q.assign(static_cast<size_t>(seq) + 1, -7);
        cu_k.assign(static_cast<size_t>(seg) + 1, -7);
        cu_pages.assign(static_cast<size_t>(seg) + 1, -7);
        page_list.assign(static_cast<size_t>(pages), -7);
        pairs.assign(static_cast<size_t>(seg), -7);
        work.assign(static_cast<size_t>(units) * SEGKV_UNIT_FIELDS, -7);
        merge.assign(static_cast<size_t>(merges) * SEGKV_MERGE_FIELDS, -7);
        retain.assign(static_cast<size_t>(seg), -7);
        t.seg_cap = seg, t.seq_cap = seq, t.page_cap = pages, t.unit_cap = units, t.merge_cap = merges;
        // exact-size vectors: an empty one hands over a null pointer with capacity 0
        t.seg_desc = seg_desc.empty() ? nullptr : seg_desc.data();
        t.cu_seqlens_q = cu_q.data();
        t.cu_seqlens_k = cu_k.data();
        t.cu_pages = cu_pages.data();
        t.page_list = page_list.empty() ? nullptr : page_list.data();
        t.pairs = pairs.empty() ? nullptr : pairs.data();
        t.work = work.empty() ? nullptr : work.data();
        t.merge = merge.empty() ? nullptr : merge.data();
        t.retain_lp = retain.empty() ? nullptr : retain.data();
    }
};

}  // namespace

int main(int argc, char **argv)
{
    const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
    const int iters = argc > 2 ? std::atoi(argv[2]) : 200;
    rng.seed(seed);
    int n_ok = 0, n_rejected = 0, n_oracle = 0;
    for (int it = 0; it < iters; ++it) {
        const int D = pick({64, 128}), P = pick({16, 32, 64, 128, 256});
        const int hkv = static_cast<int>(rnd(1, 4)), G = pick({1, 2, 4, 8}), hq = hkv * G;
        const int S = static_cast<int>(rnd(1, 6));
        const bool small = rnd(0, 3) == 0;   // small enough for the oracle
        std::vector<int32_t> c(S), n(S), win(hkv);
        std::vector<int8_t> cls(hkv);
        for (int b = 0; b < S; ++b) {
            c[b] = rnd(0, 3) == 0 ? 0 : static_cast<int32_t>(rnd(0, small ? 90 : 3000));
            n[b] = rnd(0, 3) == 0 ? static_cast<int32_t>(rnd(1, 4)) : static_cast<int32_t>(rnd(1, small ? 40 : 700));
        }
        for (int g = 0; g < hkv; ++g) {
            cls[g] = static_cast<int8_t>(rnd(0, 1));
            win[g] = pick({1, 2, static_cast<int>(rnd(1, 300)), static_cast<int>(rnd(1, 5000))});
        }
        int max_lp = 1;
        int64_t needed = 0;
        for (int b = 0; b < S; ++b) {
            const int lp = (c[b] + n[b] + P - 1) / P;
            max_lp = std::max(max_lp, lp);
            needed += static_cast<int64_t>(lp) * hkv;
        }
        const int64_t num_pages = needed + rnd(0, needed / 4 + 3);
        // page ids: a seeded permutation of the pool, -1 where nothing is stored
        std::vector<int32_t> perm(static_cast<size_t>(num_pages));
        for (int64_t i = 0; i < num_pages; ++i) perm[static_cast<size_t>(i)] = static_cast<int32_t>(i);
        std::shuffle(perm.begin(), perm.end(), rng);
        std::vector<int32_t> page_of(static_cast<size_t>(S) * hkv * max_lp, -1);
        size_t next = 0;
        for (int b = 0; b < S; ++b)
            for (int g = 0; g < hkv; ++g)
                for (int lp = 0; lp < (c[b] + n[b] + P - 1) / P; ++lp)
                    page_of[(static_cast<size_t>(b) * hkv + g) * max_lp + lp] = perm[next++];

        // one fault at most per iteration
        const int mode = static_cast<int>(rnd(0, 11));
        int expect_rc = SEGKV_OK;
        int in_max_lp = max_lp;
        if (mode == 0) {   // an id outside the pool at a position the builder must read (the last page)
            const int b = static_cast<int>(rnd(0, S - 1)), g = static_cast<int>(rnd(0, hkv - 1));
            const int lp = (c[b] + n[b] - 1) / P;
            page_of[(static_cast<size_t>(b) * hkv + g) * max_lp + lp] =
                pick({-1, -1000, static_cast<int32_t>(num_pages), static_cast<int32_t>(num_pages + 77)});
            expect_rc = SEGKV_ERR_OUT_OF_RANGE;
        } else if (mode == 1 && max_lp > 1) {   // max_lp one short of the longest sequence
            in_max_lp = max_lp - 1;
            expect_rc = SEGKV_ERR_OUT_OF_RANGE;
        } else if (mode == 2) {
            const int b = static_cast<int>(rnd(0, S - 1));
            if (rnd(0, 1)) c[b] = -static_cast<int32_t>(rnd(1, 5)); else n[b] = 0;
            expect_rc = SEGKV_ERR_INVALID_ARG;
        } else if (mode == 3) {
            const int g = static_cast<int>(rnd(0, hkv - 1));
            cls[g] = 0, win[g] = pick({0, -3});
            expect_rc = SEGKV_ERR_INVALID_ARG;
        }
        // page_of with the short max_lp: rows re-laid at the narrower stride
        std::vector<int32_t> po_in = page_of;
        if (in_max_lp != max_lp) {
            po_in.assign(static_cast<size_t>(S) * hkv * in_max_lp, -1);
            for (int s = 0; s < S * hkv; ++s)
                for (int lp = 0; lp < in_max_lp; ++lp)
                    po_in[static_cast<size_t>(s) * in_max_lp + lp] = page_of[static_cast<size_t>(s) * max_lp + lp];
        }

        segkv_config cfg{};
        cfg.num_q_heads = hq, cfg.num_kv_heads = hkv, cfg.head_dim = D, cfg.page_size = P, cfg.num_pages = num_pages;
        cfg.k_pool = reinterpret_cast<void *>(uintptr_t{1} << 32);
        cfg.v_pool = reinterpret_cast<void *>(uintptr_t{3} << 32);
        segkv_ctx *ctx = nullptr;
        if (segkv_create(&cfg, &ctx) != SEGKV_OK || !ctx) {
            expect(false, "segkv_create refused a valid configuration", it);
            continue;
        }
        segkv_table_inputs in{};
        in.num_seqs = S, in.max_lp = in_max_lp;
        in.cached_len = c.data(), in.new_len = n.data(), in.head_class = cls.data(), in.window = win.data();
        in.page_of = po_in.data();
        in.max_unit_tiles = pick({0, 0, -1, static_cast<int>(rnd(1, 6)), static_cast<int>(rnd(7, 40))});

        // first call: sizes only
        segkv_tables t{};
        int rc = segkv_build_head_tables(ctx, &in, &t);
        if (expect_rc != SEGKV_OK) {
            expect(rc == expect_rc, "bad input not refused with the expected code", it);
            ++n_rejected;
            segkv_destroy(ctx);
            continue;
        }
        expect(rc == SEGKV_ERR_CAPACITY, "size query did not report capacity", it);
        const int segs = t.num_segments, units = t.num_units, merges = t.num_merges;
        const int64_t pages = t.num_page_entries;
        expect(segs == S * hkv, "segment count", it);
        Buffers buf;
        // a buffer one short is refused
        if (rnd(0, 2) == 0 && (pages > 0 || units > 0)) {
            segkv_tables s2{};
            if (pages > 0 && rnd(0, 1)) buf.bind(s2, segs, S, pages - 1, units, merges);
            else if (units > 0) buf.bind(s2, segs, S, pages, units - 1, merges);
            else buf.bind(s2, segs, S, pages - 1, units, merges);
            expect(segkv_build_head_tables(ctx, &in, &s2) == SEGKV_ERR_CAPACITY, "short buffer accepted", it);
        }
        segkv_tables t2{};
        buf.bind(t2, segs, S, pages, units, merges);
        rc = segkv_build_head_tables(ctx, &in, &t2);
        expect(rc == SEGKV_OK, "exact buffers refused", it);
        if (rc != SEGKV_OK) {
            segkv_destroy(ctx);
            continue;
        }
        ++n_ok;
        // invariants
        int64_t pair_sum = 0;
        for (int s = 0; s < segs; ++s) pair_sum += buf.pairs[static_cast<size_t>(s)];
        expect(pair_sum == t2.total_pairs, "pairs do not sum to total_pairs", it);
        for (int b = 0; b < S; ++b)
            expect(buf.cu_q[static_cast<size_t>(b) + 1] - buf.cu_q[static_cast<size_t>(b)] == n[b], "cu_seqlens_q", it);
        for (int64_t i = 0; i < pages; ++i)
            expect(buf.page_list[static_cast<size_t>(i)] >= 0 && buf.page_list[static_cast<size_t>(i)] < num_pages,
                   "page list id outside the pool", it);
        for (int u = 0; u < units; ++u) {
            const int32_t *w = &buf.work[static_cast<size_t>(u) * SEGKV_UNIT_FIELDS];
            expect(w[SEGKV_UNIT_SEGMENT] >= 0 && w[SEGKV_UNIT_SEGMENT] < segs, "unit segment", it);
            expect(w[SEGKV_UNIT_TILES] >= 0 && w[SEGKV_UNIT_PART] >= -1 && w[SEGKV_UNIT_PART] < t2.num_parts,
                   "unit tiles / part", it);
        }
        for (int m = 0; m < merges; ++m) {
            const int32_t *e = &buf.merge[static_cast<size_t>(m) * SEGKV_MERGE_FIELDS];
            expect(e[SEGKV_MERGE_PART0] >= 0 && e[SEGKV_MERGE_NPARTS] >= 2 &&
                       e[SEGKV_MERGE_PART0] + e[SEGKV_MERGE_NPARTS] <= t2.num_parts, "merge parts", it);
        }

        // attention entry points: host-side checks before any launch
        segkv_dev_tables dt{};
        dt.seg_desc = buf.seg_desc.data(), dt.page_list = buf.page_list.data(), dt.work = buf.work.data();
        dt.num_segments = segs, dt.num_units = units, dt.num_page_entries = pages;
        dt.total_q_rows = t2.total_q_rows, dt.unit_rows = t2.unit_rows, dt.unit_heads = t2.unit_heads;
        dt.merge = merges ? buf.merge.data() : nullptr, dt.num_merges = merges, dt.num_parts = t2.num_parts;
        void *fake = reinterpret_cast<void *>(uintptr_t{5} << 32);
        expect(segkv_attn_prefill(ctx, &dt, nullptr, fake, SEGKV_DTYPE_F32, nullptr, 0.f, nullptr, 0, nullptr) ==
                   (units ? SEGKV_ERR_INVALID_ARG : SEGKV_OK), "null q accepted", it);
        expect(segkv_attn_prefill(ctx, &dt, fake, fake, 7, nullptr, 0.f, nullptr, 0, nullptr) == SEGKV_ERR_INVALID_ARG,
               "bad o_dtype accepted", it);
        if (t2.num_parts > 0) {
            expect(segkv_attn_prefill(ctx, &dt, fake, fake, SEGKV_DTYPE_F32, nullptr, 0.f, fake,
                                      t2.workspace_bytes - 1, nullptr) == SEGKV_ERR_CAPACITY,
                   "short workspace accepted", it);
        }
        rc = segkv_attn_prefill_noalloc(ctx, &dt, fake, fake, SEGKV_DTYPE_BF16, nullptr, 0.f, nullptr);
        expect(rc == (units ? (t2.workspace_bytes > SEGKV_NOALLOC_SCRATCH_BYTES ? SEGKV_ERR_CAPACITY
                                                                                 : SEGKV_ERR_UNSUPPORTED)
                            : SEGKV_OK), "no-alloc entry point", it);

        // the oracle on the builder's tables (small layers)
        int64_t rows = 0;
        for (int b = 0; b < S; ++b) rows += n[b];
        if (small && num_pages * P * D <= (int64_t{1} << 22)) {
            std::vector<uint16_t> kp(static_cast<size_t>(num_pages * P * D)), vp(kp.size());
            std::vector<uint16_t> q(static_cast<size_t>(rows * hq * D));
            for (auto &x : kp) x = static_cast<uint16_t>(0x3c00 + rnd(0, 0x7ff) - 0x400);   // |x| in ~[2^-16, 4)
            for (auto &x : vp) x = static_cast<uint16_t>(0x3c00 + rnd(0, 0x7ff) - 0x400);
            for (auto &x : q) x = static_cast<uint16_t>(0x3c00 + rnd(0, 0x7ff) - 0x400);
            std::vector<int32_t> f[8];
            for (auto &v : f) v.resize(static_cast<size_t>(segs));
            for (int s = 0; s < segs; ++s)
                for (int k = 0; k < 8; ++k) f[k][static_cast<size_t>(s)] = buf.seg_desc[static_cast<size_t>(s) * 8 + k];
            std::vector<int32_t> qs;
            for (int b = 0; b < S; ++b)
                for (int h = 0; h < hq; ++h)
                    for (int r = 0; r < n[b]; ++r) qs.insert(qs.end(), {b, h, r});
            const int64_t nq = static_cast<int64_t>(qs.size() / 3);
            std::vector<double> o(static_cast<size_t>(nq * D)), lse(static_cast<size_t>(nq));
            rc = oracle_attn_fp64(kp.data(), vp.data(), num_pages, P, D, q.data(), rows, hq, hkv, segs,
                                  f[SEGKV_SEG_Q_ROW0].data(), f[SEGKV_SEG_N_Q].data(), f[SEGKV_SEG_Q_POS0].data(),
                                  f[SEGKV_SEG_KV_HEAD].data(), f[SEGKV_SEG_WINDOW].data(),
                                  f[SEGKV_SEG_K_POS0].data(), buf.cu_pages.data(), buf.page_list.data(), pages,
                                  qs.data(), nq, 1.0 / std::sqrt(static_cast<double>(D)), o.data(), lse.data());
            expect(rc == 0, "oracle refused the builder's tables", it);
            for (double x : o) expect(std::isfinite(x), "oracle output not finite", it);
            ++n_oracle;
        }
        segkv_destroy(ctx);
    }
    std::printf("fuzz_host seed %llu: %d built, %d refused as expected, %d oracle runs, %d failures\n",
                static_cast<unsigned long long>(seed), n_ok, n_rejected, n_oracle, failures);
    return failures ? 1 : 0;
}
