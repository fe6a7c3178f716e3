// Host-side head-class page-table builder (SELECTVISIBLESTATE).
//
// RedKnot summary page, "Head-Class Sparsification" and "SegPaged Attention":
// every (layer, KV head) carries an offline class; a global head keeps the
// full causal context, a local head keeps a sliding window, and each head
// physically keeps only the pages its visible keys live in. This file turns
// one layer's class table, sequence lengths and block table (the
// logical-to-physical page map of the KV-cache management page, section 3.1)
// into the flat arrays the attention kernel reads, plus the kernel's work
// list ordered longest-first in L2-sharing cohorts.
#include <algorithm>
#include <cstring>
#include <limits>
#include <vector>

#include "segkv_internal.h"

namespace {

struct Seg {
    int32_t q_row0, n_q, q_pos0, kv_head, window, k_pos0, k_len, page_off;
    int32_t first_lp, n_pages;
    int64_t pairs;
};

// One work unit: a block (segment, row block, head block) over a run of its tiles.
struct Unit {
    int32_t seg, row0, head0, tiles, tile0, part;
};

// Sum over the n new rows i = c .. c+n-1 of the number of visible keys,
// min(i + 1, W) for a local head (W > 0) or i + 1 for a global head (W == 0).
int64_t visible_pairs(int64_t c, int64_t n, int64_t W)
{
    const int64_t a = c + 1;  // visible keys of the first new row, before the window cap
    if (W == 0) return n * a + n * (n - 1) / 2;
    if (a >= W) return n * W;
    const int64_t k = std::min<int64_t>(n, W - a);  // rows still below the cap
    return k * a + k * (k - 1) / 2 + (n - k) * W;
}

}  // namespace

extern "C" int segkv_build_head_tables(const segkv_ctx *ctx, const segkv_table_inputs *in, segkv_tables *out)
{
    using segkv::fail;
    segkv::clear_error();
    if (!ctx || !in || !out) return fail(SEGKV_ERR_INVALID_ARG, "build_head_tables: null argument");
    const segkv_config &cfg = ctx->cfg;
    const int32_t hq = cfg.num_q_heads, hkv = cfg.num_kv_heads, P = cfg.page_size;
    const int32_t G = hq / hkv;
    const int32_t S = in->num_seqs;
    if (S < 1) return fail(SEGKV_ERR_INVALID_ARG, "build_head_tables: num_seqs must be >= 1");
    if (in->max_lp < 1) return fail(SEGKV_ERR_INVALID_ARG, "build_head_tables: max_lp must be >= 1");
    if (!in->cached_len || !in->new_len || !in->head_class || !in->window || !in->page_of)
        return fail(SEGKV_ERR_INVALID_ARG, "build_head_tables: null input array");
    if (static_cast<int64_t>(S) * hkv > std::numeric_limits<int32_t>::max())
        return fail(SEGKV_ERR_INVALID_ARG, "build_head_tables: too many segments");

    int max_new = 0;
    for (int32_t b = 0; b < S; ++b) max_new = std::max(max_new, in->new_len[b]);
    const bool decode = segkv::decode_units(G, P, max_new);
    // Mean visible keys per query row and KV head: long contexts get
    // eight-wave units (a heuristic, summed in double; the inputs are
    // validated below, and invalid ones are skipped here).
    double vis_keys = 0.0, vis_rows = 0.0;
    for (int32_t b = 0; b < S; ++b) {
        const int64_t c = in->cached_len[b], n = in->new_len[b];
        if (c < 0 || n < 1 || c > std::numeric_limits<int32_t>::max() || n > std::numeric_limits<int32_t>::max())
            continue;
        for (int32_t g = 0; g < hkv; ++g) {
            const bool global = in->head_class[g] != 0;
            const int64_t W = global ? 0 : in->window[g];
            if (!global && W < 1) continue;
            vis_keys += static_cast<double>(visible_pairs(c, n, W));
            vis_rows += static_cast<double>(n);
        }
    }
    const int waves =
        segkv::unit_waves(P, vis_rows > 0.0 &&
                                    vis_keys >= static_cast<double>(segkv::wide_min_keys(cfg.head_dim)) * vis_rows);
    const segkv::UnitShape shape = decode ? segkv::decode_shape(G) : segkv::unit_shape(G, waves);
    std::vector<Seg> segs;
    segs.reserve(static_cast<size_t>(S) * hkv);
    int64_t q_rows = 0, pages = 0, units = 0, total_pairs = 0;

    for (int32_t b = 0; b < S; ++b) {
        const int64_t c = in->cached_len[b], n = in->new_len[b];
        if (c < 0 || n < 1)
            return fail(SEGKV_ERR_INVALID_ARG, "sequence %d: need cached_len >= 0 and new_len >= 1", b);
        const int64_t T = c + n;
        if (T > std::numeric_limits<int32_t>::max() || q_rows + n > std::numeric_limits<int32_t>::max())
            return fail(SEGKV_ERR_INVALID_ARG, "sequence %d: length overflows int32", b);
        for (int32_t g = 0; g < hkv; ++g) {
            Seg sg{};
            const bool global = in->head_class[g] != 0;
            int64_t first_pos = 0;
            if (!global) {
                const int64_t W = in->window[g];
                if (W < 1) return fail(SEGKV_ERR_INVALID_ARG, "kv head %d: local window must be >= 1", g);
                first_pos = (std::max<int64_t>(0, c - W + 1) / P) * P;
                sg.window = static_cast<int32_t>(W);
            }
            const int64_t first_lp = first_pos / P, last_lp = (T - 1) / P;
            if (last_lp >= in->max_lp)
                return fail(SEGKV_ERR_OUT_OF_RANGE, "sequence %d needs logical page %lld >= max_lp %d", b,
                            static_cast<long long>(last_lp), in->max_lp);
            const int32_t *row = in->page_of + (static_cast<int64_t>(b) * hkv + g) * in->max_lp;
            for (int64_t lp = first_lp; lp <= last_lp; ++lp) {
                const int32_t id = row[lp];
                if (id < 0 || id >= cfg.num_pages)
                    return fail(SEGKV_ERR_OUT_OF_RANGE, "segment (seq %d, kv head %d) logical page %lld: id %d "
                                "outside [0, %lld)", b, g, static_cast<long long>(lp), id,
                                static_cast<long long>(cfg.num_pages));
            }
            sg.q_row0 = static_cast<int32_t>(q_rows);
            sg.n_q = static_cast<int32_t>(n);
            sg.q_pos0 = static_cast<int32_t>(c);
            sg.kv_head = g;
            sg.k_pos0 = static_cast<int32_t>(first_pos);
            sg.k_len = static_cast<int32_t>(T - first_pos);
            sg.page_off = static_cast<int32_t>(pages);
            sg.first_lp = static_cast<int32_t>(first_lp);
            sg.n_pages = static_cast<int32_t>(last_lp - first_lp + 1);
            sg.pairs = G * visible_pairs(c, n, sg.window);
            pages += sg.n_pages;
            if (pages > std::numeric_limits<int32_t>::max())
                return fail(SEGKV_ERR_INVALID_ARG, "build_head_tables: page list exceeds int32 offsets");
            total_pairs += sg.pairs;
            units += ((n + shape.rows - 1) / shape.rows) * (G / shape.heads);
            segs.push_back(sg);
        }
        q_rows += n;
    }
    if (units > std::numeric_limits<int32_t>::max())
        return fail(SEGKV_ERR_INVALID_ARG, "build_head_tables: too many work units");

    // Blocks: every (segment, row block, head block) once, with the run of
    // 64-key tiles its rows see (tile0 counted from the segment's k_pos0).
    std::vector<Unit> list;
    list.reserve(static_cast<size_t>(units));
    int64_t total_tiles = 0, longest = 0;
    for (int32_t s = 0; s < static_cast<int32_t>(segs.size()); ++s) {
        const Seg &sg = segs[s];
        for (int32_t r0 = 0; r0 < sg.n_q; r0 += shape.rows) {
            const int64_t first = static_cast<int64_t>(sg.q_pos0) + r0;
            const int64_t last = static_cast<int64_t>(sg.q_pos0) + std::min(r0 + shape.rows, sg.n_q) - 1;
            const int64_t lo = sg.window == 0 ? 0 : std::max<int64_t>(0, first - sg.window + 1);
            const int64_t kbeg = lo - sg.k_pos0, kend = last + 1 - sg.k_pos0;
            const int32_t tile0 = static_cast<int32_t>(kbeg / segkv::kKvTile);
            const int32_t tiles = static_cast<int32_t>((kend + segkv::kKvTile - 1) / segkv::kKvTile) - tile0;
            for (int32_t h = 0; h < G; h += shape.heads) {
                list.push_back(Unit{s, r0, sg.kv_head * G + h, tiles, tile0, -1});
                total_tiles += tiles;
                longest = std::max<int64_t>(longest, tiles);
            }
        }
    }

    // Split-KV: cut long blocks into runs when list scheduling alone could not
    // balance them (a block longer than the mean load of a workgroup slot
    // finishes after everything else however the list is ordered).
    int64_t max_run = 0;   // 0: no split
    if (P >= segkv::kKvTile && in->max_unit_tiles >= 0) {
        if (in->max_unit_tiles > 0) {
            max_run = in->max_unit_tiles;
        } else if (decode) {
            // Decode: a handful of long blocks; cut them into enough even runs
            // for several units per workgroup slot.
            const int64_t target = static_cast<int64_t>(segkv::kDecodeSlots) * segkv::kDecodeUnitsPerSlot;
            max_run = std::max<int64_t>(segkv::kDecodeMinRun, (total_tiles + target - 1) / target);
        } else {
            const int64_t slots = static_cast<int64_t>(segkv::kXcds) * segkv::cohort(waves);
            // Runs of half a slot's mean load; the two-block kernel (head dim
            // 128, 256-pair units), whose workgroups take units from queues
            // until none is left, balances whole ones, and every extra run
            // costs it a unit's start and end: runs of a slot's mean load.
            const int64_t per = cfg.head_dim == 128 && waves == segkv::kWideWaves ? slots : 2 * slots;
            if (4 * longest * slots > 3 * total_tiles)
                max_run = std::max<int64_t>(segkv::kMinRun, (total_tiles + per - 1) / per);
        }
    }
    std::vector<int32_t> merges;   // [num_merges][SEGKV_MERGE_FIELDS]
    int64_t n_parts = 0;
    if (max_run > 0 && longest > max_run) {
        std::vector<Unit> cut;
        cut.reserve(list.size());
        for (const Unit &u : list) {
            if (u.tiles <= max_run) {
                cut.push_back(u);
                continue;
            }
            const int64_t nr = (u.tiles + max_run - 1) / max_run;
            const Seg &sg = segs[static_cast<size_t>(u.seg)];
            const int32_t merge[SEGKV_MERGE_FIELDS] = {u.seg, u.row0, u.head0, static_cast<int32_t>(n_parts),
                                                       static_cast<int32_t>(nr), sg.q_row0 + u.row0,
                                                       std::min(shape.rows, sg.n_q - u.row0), 0};
            merges.insert(merges.end(), merge, merge + SEGKV_MERGE_FIELDS);
            for (int64_t r = 0; r < nr; ++r) {   // runs of near-equal length
                const int64_t a = u.tiles * r / nr, b = u.tiles * (r + 1) / nr;
                cut.push_back(Unit{u.seg, u.row0, u.head0, static_cast<int32_t>(b - a),
                                   static_cast<int32_t>(u.tile0 + a), static_cast<int32_t>(n_parts + r)});
            }
            n_parts += nr;
        }
        list.swap(cut);
        if (static_cast<int64_t>(list.size()) > std::numeric_limits<int32_t>::max() ||
            n_parts > std::numeric_limits<int32_t>::max())
            return fail(SEGKV_ERR_INVALID_ARG, "build_head_tables: too many split units");
    }
    units = static_cast<int64_t>(list.size());
    const int32_t n_merges = static_cast<int32_t>(merges.size() / SEGKV_MERGE_FIELDS);

    const int32_t nseg = static_cast<int32_t>(segs.size());
    out->num_segments = nseg;
    out->num_units = static_cast<int32_t>(units);
    out->num_page_entries = pages;
    out->total_pairs = total_pairs;
    out->total_q_rows = static_cast<int32_t>(q_rows);
    out->unit_rows = shape.rows;
    out->unit_heads = shape.heads;
    out->num_merges = n_merges;
    out->num_parts = static_cast<int32_t>(n_parts);
    out->workspace_bytes = SEGKV_WORKSPACE_BYTES(n_parts, shape.rows, shape.heads, cfg.head_dim);
    if (out->seg_cap < nseg || out->seq_cap < S || out->page_cap < pages || out->unit_cap < units ||
        out->merge_cap < n_merges)
        return fail(SEGKV_ERR_CAPACITY, "build_head_tables: buffers too small (need %d segments, %d sequences, "
                    "%lld page entries, %lld units, %d merges)", nseg, S, static_cast<long long>(pages),
                    static_cast<long long>(units), n_merges);
    if (!out->seg_desc || !out->cu_seqlens_q || !out->cu_seqlens_k || !out->cu_pages || !out->page_list ||
        !out->pairs || !out->work || (n_merges > 0 && !out->merge))
        return fail(SEGKV_ERR_INVALID_ARG, "build_head_tables: null output buffer");

    // Segment arrays, prefix sums and the page list.
    int64_t k_acc = 0;
    out->cu_seqlens_k[0] = 0;
    out->cu_pages[0] = 0;
    for (int32_t s = 0; s < nseg; ++s) {
        const Seg &sg = segs[s];
        int32_t *d = out->seg_desc + static_cast<int64_t>(s) * SEGKV_SEG_FIELDS;
        d[SEGKV_SEG_Q_ROW0] = sg.q_row0;
        d[SEGKV_SEG_N_Q] = sg.n_q;
        d[SEGKV_SEG_Q_POS0] = sg.q_pos0;
        d[SEGKV_SEG_KV_HEAD] = sg.kv_head;
        d[SEGKV_SEG_WINDOW] = sg.window;
        d[SEGKV_SEG_K_POS0] = sg.k_pos0;
        d[SEGKV_SEG_K_LEN] = sg.k_len;
        d[SEGKV_SEG_PAGE_OFF] = sg.page_off;
        k_acc += sg.k_len;
        if (k_acc > std::numeric_limits<int32_t>::max())
            return fail(SEGKV_ERR_INVALID_ARG, "build_head_tables: cu_seqlens_k overflows int32");
        out->cu_seqlens_k[s + 1] = static_cast<int32_t>(k_acc);
        out->cu_pages[s + 1] = sg.page_off + sg.n_pages;
        out->pairs[s] = sg.pairs;
        if (out->retain_lp) {
            const int64_t T = static_cast<int64_t>(sg.q_pos0) + sg.n_q;
            out->retain_lp[s] = sg.window == 0 ? 0 : static_cast<int32_t>(std::max<int64_t>(0, T - sg.window + 1) / P);
        }
        const int32_t *row = in->page_of + static_cast<int64_t>(s) * in->max_lp;
        std::memcpy(out->page_list + sg.page_off, row + sg.first_lp, sizeof(int32_t) * sg.n_pages);
    }
    out->cu_seqlens_q[0] = 0;
    for (int32_t b = 0; b < S; ++b) out->cu_seqlens_q[b + 1] = out->cu_seqlens_q[b] + in->new_len[b];

    // Work list: longest first, then dealt to the XCDs in cohorts.
    std::stable_sort(list.begin(), list.end(), [](const Unit &a, const Unit &b) { return a.tiles > b.tiles; });

    // Cohorts for the L2 caches. Workgroups go to the XCDs round-robin by
    // index, and each XCD has its own L2. Consecutive windows of the sorted
    // list (units of similar cost) are re-dealt so that every XCD receives
    // neighbouring units in (segment, row) order: they start together and
    // walk the same K/V tiles at about the same time, so one L2 fill serves
    // them all instead of each unit refetching its window from HBM.
    const size_t n_units = list.size();
    const size_t window = static_cast<size_t>(segkv::kXcds) * (decode ? segkv::kCohort : segkv::cohort(waves));
    std::vector<Unit> dealt(n_units);
    for (size_t base = 0; base < n_units; base += window) {
        const size_t n = std::min(window, n_units - base);
        std::sort(list.begin() + base, list.begin() + base + n, [](const Unit &a, const Unit &b) {
            if (a.seg != b.seg) return a.seg < b.seg;
            if (a.row0 != b.row0) return a.row0 < b.row0;
            if (a.head0 != b.head0) return a.head0 < b.head0;
            return a.tile0 < b.tile0;
        });
        // Positions base + 8j + x belong to XCD x. The XCDs take the sorted
        // window in turn, in reverse turn order every other window, so that
        // no XCD always receives the costlier end of the windows (each XCD
        // drains only its own share of the list). Each XCD's share is laid
        // out last row first: a causal head's later rows are its longer
        // units, and the workgroups of an XCD take their next unit in the
        // order they finish, so the one that finished first (the shortest
        // unit) takes the longest next one. In ascending order the early
        // finishers took the shortest again and the XCD's units drifted apart
        // in the K/V stream over the launch (by ~200 tiles, more than the L2
        // holds, at a 128K layer's end), and each refetched it.
        const bool reverse = (base / window) % 2 == 1;
        size_t idx = 0;
        for (int t = 0; t < segkv::kXcds; ++t) {
            const int x = reverse ? segkv::kXcds - 1 - t : t;
            const size_t c = static_cast<size_t>(x) < n ? (n - x + segkv::kXcds - 1) / segkv::kXcds : 0;
            for (size_t k = 0; k < c; ++k) dealt[base + x + k * segkv::kXcds] = list[base + idx + c - 1 - k];
            idx += c;
        }
    }
    for (size_t u = 0; u < n_units; ++u) {
        int32_t *w = out->work + u * SEGKV_UNIT_FIELDS;
        w[SEGKV_UNIT_SEGMENT] = dealt[u].seg;
        w[SEGKV_UNIT_ROW0] = dealt[u].row0;
        w[SEGKV_UNIT_HEAD0] = dealt[u].head0;
        w[SEGKV_UNIT_TILES] = dealt[u].tiles;
        w[SEGKV_UNIT_TILE0] = dealt[u].tile0;
        w[SEGKV_UNIT_PART] = dealt[u].part;
        const Seg &sg = segs[dealt[u].seg];
        for (int i = 0; i < 4; ++i) {
            const int64_t lp = (static_cast<int64_t>(dealt[u].tile0) + i) * segkv::kKvTile / P;
            w[SEGKV_UNIT_PAGE0 + i] =
                i < dealt[u].tiles && lp < sg.n_pages ? out->page_list[sg.page_off + lp] : -1;
        }
        w[10] = 0;
        w[11] = 0;
    }
    if (n_merges > 0) std::memcpy(out->merge, merges.data(), sizeof(int32_t) * merges.size());
    return SEGKV_OK;
}
