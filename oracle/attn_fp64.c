/*
 * Oracle: fp64 head-segmented paged prefill attention on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and
 * bench.py's cpu_baseline leg may load this library. It shares no code,
 * header or constant with the HIP library under test.
 *
 * What it computes (RedKnot summary page, "SegPaged Attention" and
 * "Head-Class Sparsification" sections; the head-split page states that
 * splitting per head leaves the result identical to the unsplit mechanism):
 * exact causal / sliding-window softmax attention, evaluated per query over
 * the query's visible key set, reading each key and value through the
 * segment's page list.
 *
 *   for query head h, KV head g = h / G, query at absolute position i:
 *     visible keys  V(i) = { j : lo(i) <= j <= i },
 *                   lo(i) = 0 for a global head, max(0, i - W + 1) for a local one
 *     s_j  = scale * sum_d q[i,h,d] * k[j,g,d]
 *     m    = max_{j in V(i)} s_j
 *     O[i,h,:] = sum_j exp(s_j - m) v[j,g,:] / sum_j exp(s_j - m)
 *     lse  = m + log(sum_j exp(s_j - m))
 *
 * It is the plain two-pass definition (not an online softmax). Every bf16
 * input is widened exactly to double; all arithmetic is double.
 *
 * Pool layout read here (the storage contract of the library):
 *   K pool: bf16 [num_pages][P][D]   (slot-major: one key's D values contiguous)
 *   V pool: bf16 [num_pages][D][P]   (dim-major:  one dim's P slot values contiguous)
 * Key position j of a segment lives in the page at index
 * (j / P - k_pos0 / P) of the segment's page list, slot j % P.
 *
 * oracle_mass_fp64 adds the attention mass each new token receives (RedKnot
 * summary page, "Sparse FFN": only the tokens with the highest attention
 * scores go through the dense FFN). Reading taken: the mass of the token at
 * position j is the sum, over every query row of the step and every query
 * head, of its softmax weight on j:
 *   mass[j] = sum_h sum_{i : j in V(i)} exp(s_j(i) - lse(i))
 * kept for the step's own (new) tokens j >= c_b.
 *
 * Pins (tests/test_oracle_attn.py): brute-force dense attention with an
 * explicit boolean mask; closed forms (first row = v_0, W = 1 gives v_i,
 * Q = 0 gives the mean of exactly the visible rows, constant V); torch's
 * fp64 causal SDPA for global heads; invariants (W >= T equals global,
 * physical page relabelling, chunked equals monolithic).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the oracle's parallel loop runs on. */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the threads of the parallel loop (a single-thread timing); n < 1 is ignored. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Returns 0 on success, 1 on a bad argument, 2 on an index out of range. */
int oracle_attn_fp64(const uint16_t *k_pool, const uint16_t *v_pool, int64_t num_pages,
                     int32_t P, int32_t D,
                     const uint16_t *q, int64_t q_rows, int32_t hq, int32_t hkv,
                     int32_t num_segments,
                     const int32_t *q_row0, const int32_t *n_q, const int32_t *q_pos0,
                     const int32_t *kv_head, const int32_t *window, const int32_t *k_pos0,
                     const int32_t *cu_pages, const int32_t *page_list, int64_t page_list_len,
                     const int32_t *queries, int64_t num_queries, /* [num_queries][3]: b, h, t */
                     double scale, double *o, double *lse)
{
    if (P <= 0 || D <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0)
        return 1;
    const int32_t G = hq / hkv;
    int status = 0;
#define FAIL()                  \
    do {                        \
        _Pragma("omp atomic write") \
        status = 2;             \
    } while (0)

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t x = 0; x < num_queries; ++x) {
        const int32_t b = queries[3 * x + 0];
        const int32_t h = queries[3 * x + 1];
        const int32_t t = queries[3 * x + 2];
        if (h < 0 || h >= hq) { FAIL(); continue; }
        const int32_t g = h / G;                 /* contiguous GQA groups */
        const int64_t s = (int64_t)b * hkv + g;  /* segment of (sequence b, KV head g) */
        if (b < 0 || s >= num_segments || kv_head[s] != g || t < 0 || t >= n_q[s]) {
            FAIL();
            continue;
        }
        const int64_t row = (int64_t)q_row0[s] + t;
        if (row >= q_rows) { FAIL(); continue; }
        const int64_t i = (int64_t)q_pos0[s] + t;
        const int64_t lo = window[s] == 0 ? 0 : (i - window[s] + 1 > 0 ? i - window[s] + 1 : 0);
        const int64_t first_lp = k_pos0[s] / P;
        const uint16_t *qrow = q + (row * hq + h) * (int64_t)D;

        double *score = (double *)malloc(sizeof(double) * (size_t)(i - lo + 1));
        int bad = 0;
        /* pass 1: scores and their maximum */
        double m = -INFINITY;
        for (int64_t j = lo; j <= i; ++j) {
            int64_t e = (int64_t)cu_pages[s] + (j / P - first_lp);
            if (j < k_pos0[s] || e >= cu_pages[s + 1] || e >= page_list_len) { bad = 1; break; }
            int64_t page = page_list[e];
            if (page < 0 || page >= num_pages) { bad = 1; break; }
            const uint16_t *krow = k_pool + (page * P + j % P) * (int64_t)D;
            double dot = 0.0;
            for (int32_t d = 0; d < D; ++d)
                dot += widen_bf16(qrow[d]) * widen_bf16(krow[d]);
            score[j - lo] = scale * dot;
            if (score[j - lo] > m) m = score[j - lo];
        }
        if (bad) { free(score); FAIL(); continue; }

        /* pass 2: normalised weighted sum of the visible values */
        double *out = o + x * (int64_t)D;
        for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
        double denom = 0.0;
        for (int64_t j = lo; j <= i; ++j) {
            int64_t page = page_list[(int64_t)cu_pages[s] + (j / P - first_lp)];
            double p = exp(score[j - lo] - m);
            denom += p;
            const uint16_t *vpage = v_pool + page * (int64_t)D * P;
            for (int32_t d = 0; d < D; ++d)
                out[d] += p * widen_bf16(vpage[(int64_t)d * P + j % P]);
        }
        for (int32_t d = 0; d < D; ++d) out[d] /= denom;
        if (lse) lse[x] = m + log(denom);
        free(score);
    }
#undef FAIL
    return status;
}

/* Attention mass of the new tokens (see the header). mass: double [q_rows],
 * zeroed here; queries as for oracle_attn_fp64 (normally every (b, h, t)). */
int oracle_mass_fp64(const uint16_t *k_pool, int64_t num_pages, int32_t P, int32_t D,
                     const uint16_t *q, int64_t q_rows, int32_t hq, int32_t hkv, int32_t num_segments,
                     const int32_t *q_row0, const int32_t *n_q, const int32_t *q_pos0,
                     const int32_t *kv_head, const int32_t *window, const int32_t *k_pos0,
                     const int32_t *cu_pages, const int32_t *page_list, int64_t page_list_len,
                     const int32_t *queries, int64_t num_queries, double scale, double *mass)
{
    if (P <= 0 || D <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0)
        return 1;
    const int32_t G = hq / hkv;
    int status = 0;
    for (int64_t r = 0; r < q_rows; ++r) mass[r] = 0.0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t x = 0; x < num_queries; ++x) {
        const int32_t b = queries[3 * x + 0], h = queries[3 * x + 1], t = queries[3 * x + 2];
        const int32_t g = (h >= 0 && h < hq) ? h / G : -1;
        const int64_t s = (int64_t)b * hkv + g;
        if (g < 0 || b < 0 || s >= num_segments || kv_head[s] != g || t < 0 || t >= n_q[s] ||
            (int64_t)q_row0[s] + t >= q_rows) {
#pragma omp atomic write
            status = 2;
            continue;
        }
        const int64_t i = (int64_t)q_pos0[s] + t;
        const int64_t lo = window[s] == 0 ? 0 : (i - window[s] + 1 > 0 ? i - window[s] + 1 : 0);
        const int64_t first_lp = k_pos0[s] / P;
        const uint16_t *qrow = q + (((int64_t)q_row0[s] + t) * hq + h) * (int64_t)D;
        double *score = (double *)malloc(sizeof(double) * (size_t)(i - lo + 1));
        int bad = 0;
        double m = -INFINITY;
        for (int64_t j = lo; j <= i; ++j) {
            int64_t e = (int64_t)cu_pages[s] + (j / P - first_lp);
            if (j < k_pos0[s] || e >= cu_pages[s + 1] || e >= page_list_len) { bad = 1; break; }
            int64_t page = page_list[e];
            if (page < 0 || page >= num_pages) { bad = 1; break; }
            const uint16_t *krow = k_pool + (page * P + j % P) * (int64_t)D;
            double dot = 0.0;
            for (int32_t d = 0; d < D; ++d) dot += widen_bf16(qrow[d]) * widen_bf16(krow[d]);
            score[j - lo] = scale * dot;
            if (score[j - lo] > m) m = score[j - lo];
        }
        if (bad) {
            free(score);
#pragma omp atomic write
            status = 2;
            continue;
        }
        double denom = 0.0;
        for (int64_t j = lo; j <= i; ++j) denom += exp(score[j - lo] - m);
        const double lse = m + log(denom);
        for (int64_t j = lo > q_pos0[s] ? lo : q_pos0[s]; j <= i; ++j) {
            const double p = exp(score[j - lo] - lse);
#pragma omp atomic
            mass[(int64_t)q_row0[s] + (j - q_pos0[s])] += p;
        }
        free(score);
    }
    return status;
}
