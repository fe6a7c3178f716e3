/*
 * segkv — head-segmented paged KV cache and fused variable-length prefill
 * attention for AMD Instinct MI355X (gfx950).
 *
 * The method (RedKnot summary page, sections "Head-Class Sparsification" and
 * "SegPaged Attention"): instead of one dense [B, H, L, D] tensor, the KV
 * cache is stored as fixed-size pages segmented per (layer, KV head). Each
 * (layer, KV head) is labelled offline as global (keeps and attends to the
 * full causal context) or local (keeps and attends to a sliding window).
 * A single fused variable-length attention pass then runs causal prefill
 * over every head's visible key set, with no attention-mask tensor. The same
 * page records the runtime's adapter split; this library provides three of
 * them:
 *   BUILDSTATE          -> segkv_write_pages       (paged KV write)
 *   SELECTVISIBLESTATE  -> segkv_build_head_tables (per-head page tables)
 *   EXECUTE             -> segkv_attn_prefill      (fused varlen attention)
 * Fixed-size pages with a logical-to-physical map are the PagedAttention
 * scheme summarised on the KV-cache management page (section 3.1).
 *
 * Definitions used throughout
 *   S sequences b = 0..S-1, each with c_b cached tokens (positions
 *   0..c_b-1, already in the pool) and n_b >= 1 new tokens (positions
 *   c_b..T_b-1, T_b = c_b + n_b) whose queries are computed.
 *   hq query heads, hkv KV heads, G = hq / hkv; query head h reads KV head
 *   h / G (contiguous GQA groups).
 *   A local head with window W lets query position i see keys j with
 *   i - W < j <= i (the W newest keys, itself included); a global head lets
 *   it see 0 <= j <= i.
 *   One layer's segments are s = b * hkv + g.
 *
 * Ownership and execution model
 *   The caller owns every device buffer (pools, Q, O, LSE, device copies of
 *   the tables). The library never allocates or frees device memory and never
 *   synchronises: GPU work is enqueued on the caller's hipStream_t, passed as
 *   void* (NULL = the null stream). A context holds only a host copy of its
 *   configuration. Functions are thread-safe except that a context must not
 *   be destroyed while in use.
 *
 * Errors
 *   Every int-returning call returns SEGKV_OK (0) or a negative code below;
 *   segkv_last_error() then returns a thread-local message. All argument
 *   checks run on the host before anything is enqueued. Device-side metadata
 *   (page ids, row offsets) is bounds-checked inside the kernels: an entry
 *   out of range is skipped (write) or read as zeros (attention), never
 *   dereferenced.
 */
#ifndef SEGKV_H
#define SEGKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    SEGKV_OK = 0,
    SEGKV_ERR_INVALID_ARG = -1,  /* null pointer, bad size, n_b < 1, W < 1, hq % hkv != 0 ... */
    SEGKV_ERR_OUT_OF_RANGE = -2, /* a page id needed by a visible range is -1 or >= num_pages */
    SEGKV_ERR_CAPACITY = -3,     /* an output buffer is too small; required sizes written back */
    SEGKV_ERR_HIP = -4,          /* a HIP launch failed; the message holds HIP's error string */
    SEGKV_ERR_UNSUPPORTED = -5   /* head_dim or page_size the kernels are not built for */
};

enum { SEGKV_DTYPE_F32 = 0, SEGKV_DTYPE_BF16 = 1 };

/* Fields of one segment descriptor (int32 [num_segments][SEGKV_SEG_FIELDS]). */
enum {
    SEGKV_SEG_Q_ROW0 = 0,   /* first row of this sequence in Q / O */
    SEGKV_SEG_N_Q = 1,      /* n_b, query rows of the sequence */
    SEGKV_SEG_Q_POS0 = 2,   /* c_b, absolute position of query row 0 */
    SEGKV_SEG_KV_HEAD = 3,  /* g; the segment serves query heads g*G .. g*G+G-1 */
    SEGKV_SEG_WINDOW = 4,   /* W for a local head, 0 for a global head */
    SEGKV_SEG_K_POS0 = 5,   /* absolute position of the segment's first stored key (page aligned) */
    SEGKV_SEG_K_LEN = 6,    /* T_b - k_pos0 keys stored for the segment */
    SEGKV_SEG_PAGE_OFF = 7, /* offset of the segment's first page id in page_list */
    SEGKV_SEG_FIELDS = 8
};

/* Fields of one work unit (int32 [num_units][SEGKV_UNIT_FIELDS]). A unit is
 * one workgroup of the attention kernel: unit_rows consecutive query rows of
 * one segment for unit_heads consecutive query heads of its GQA group, over
 * a run of the 64-key tiles those rows see. The builder picks the shape per
 * call: unit_rows * unit_heads = 128 for short contexts, 256 for long ones
 * with pages >= 64 (a mean of at least 1024 visible keys per query row and KV
 * head at head dim 128, 2048 at 64), or 32 / G rows x G heads for decode
 * steps. A block
 * whose run is split into several units (split-KV) writes partial results to
 * the workspace, and one merge entry per block combines them. */
enum {
    SEGKV_UNIT_SEGMENT = 0,
    SEGKV_UNIT_ROW0 = 1,    /* first query row, relative to the segment (0 .. n_b-1) */
    SEGKV_UNIT_HEAD0 = 2,   /* first query head (absolute) */
    SEGKV_UNIT_TILES = 3,   /* KV tiles the unit visits: its cost, used to order the list */
    SEGKV_UNIT_TILE0 = 4,   /* first tile, counted in 64-key steps from the segment's k_pos0 */
    SEGKV_UNIT_PART = 5,    /* workspace slot of a split unit's partial result, -1 = writes O */
    SEGKV_UNIT_PAGE0 = 6,   /* fields 6 .. 9: page ids of the unit's tiles tile0 .. tile0+3 (-1 past its
                               run or past the segment's pages), copies of page-list entries: the
                               kernels start their first K/V transfers from them without first
                               reading the page list */
    SEGKV_UNIT_FIELDS = 12  /* fields 10, 11 are zero */
};

/* Fields of one merge entry (int32 [num_merges][SEGKV_MERGE_FIELDS]): the
 * block of a split unit and its partial results, workspace slots
 * part0 .. part0 + nparts - 1. */
enum {
    SEGKV_MERGE_SEGMENT = 0,
    SEGKV_MERGE_ROW0 = 1,
    SEGKV_MERGE_HEAD0 = 2,
    SEGKV_MERGE_PART0 = 3,
    SEGKV_MERGE_NPARTS = 4,
    SEGKV_MERGE_OUT_ROW0 = 5,   /* first output row of the block: the segment's q_row0 + row0 */
    SEGKV_MERGE_ROWS = 6,       /* rows of the block that exist: min(unit_rows, n_b - row0) */
    SEGKV_MERGE_FIELDS = 8      /* field 7 is zero */
};

/* Workspace bytes per partial result: the unit's unit_rows * unit_heads
 * (query row, head) pairs, each with head_dim unnormalised fp32 outputs plus
 * its running maximum and sum. */
#define SEGKV_PART_BYTES(unit_rows, unit_heads, head_dim) \
    (4 * (int64_t)(unit_rows) * (int64_t)(unit_heads) * ((int64_t)(head_dim) + 2))

/* Bytes after the partial results in the workspace of tables whose units
 * hold 256 (row, head) pairs: the work queues of the persistent attention
 * kernel (eight per-XCD unit counters, zeroed by each call on its stream). */
#define SEGKV_QUEUE_BYTES 256

/* The workspace segkv_attn_prefill needs (the builder's workspace_bytes). */
#define SEGKV_WORKSPACE_BYTES(num_parts, unit_rows, unit_heads, head_dim)                      \
    ((int64_t)(num_parts) * SEGKV_PART_BYTES(unit_rows, unit_heads, head_dim) +                 \
     ((int64_t)(unit_rows) * (int64_t)(unit_heads) == 256 ? (int64_t)SEGKV_QUEUE_BYTES : 0))

typedef struct segkv_ctx segkv_ctx;

/*
 * Pool layout (one pool shared by every layer, sequence and KV head):
 *   k_pool: bf16 [num_pages][page_size][head_dim]  one key's head_dim values contiguous
 *   v_pool: bf16 [num_pages][head_dim][page_size]  one dimension's page_size values contiguous
 * Position j of a segment lives at slot j % page_size of a page. Both layouts
 * make one page a single contiguous block (16 KiB for P = 64, D = 128); the
 * transposed V page puts the key index innermost, which is the order the
 * P.V contraction consumes it in.
 */
typedef struct segkv_config {
    int32_t num_q_heads;   /* hq */
    int32_t num_kv_heads;  /* hkv, hq % hkv == 0 */
    int32_t head_dim;      /* D: 64 or 128 */
    int32_t page_size;     /* P: 16, 32, 64, 128 or 256 */
    int64_t num_pages;     /* pool capacity in pages */
    void *k_pool;          /* device */
    void *v_pool;          /* device */
} segkv_config;

/* Validate cfg and return a new context in *out (host memory only). */
int segkv_create(const segkv_config *cfg, segkv_ctx **out);
void segkv_destroy(segkv_ctx *ctx);

/*
 * BUILDSTATE: scatter new K/V rows of one layer into their pages.
 *   k_new, v_new : device bf16 [num_rows][hkv][head_dim]
 *   cu_rows      : device int32 [num_seqs+1]; rows cu_rows[b] .. cu_rows[b+1]-1
 *                  belong to sequence b
 *   pos0         : device int32 [num_seqs]; absolute position of row cu_rows[b]
 *   page_of      : device int32 [num_seqs][hkv][max_lp]; physical page of each
 *                  logical page (position / page_size) of this layer, -1 none
 *   max_rows_per_seq : host bound on cu_rows[b+1]-cu_rows[b] (sizes the grid)
 * Row r of sequence b, KV head g, goes to page page_of[b][g][p / P], slot
 * p % P, p = pos0[b] + r - cu_rows[b]; K as one contiguous row of the page,
 * V into column p % P of the transposed page. Slots not written keep their
 * contents. A row whose page id is -1, >= num_pages or whose logical page is
 * >= max_lp, or whose row index is >= num_rows, is skipped.
 */
int segkv_write_pages(const segkv_ctx *ctx, const void *k_new, const void *v_new, int64_t num_rows,
                      const int32_t *cu_rows, const int32_t *pos0, const int32_t *page_of,
                      int32_t num_seqs, int32_t max_lp, int32_t max_rows_per_seq, void *stream);

/*
 * SELECTVISIBLESTATE: build one layer's per-(sequence, KV head) segment
 * tables on the host. All pointers are host memory.
 *
 * For segment s = b*hkv + g:
 *   global head: k_pos0 = 0
 *   local head:  k_pos0 = floor(max(0, c_b - W + 1) / P) * P, the start of the
 *                page holding the first key visible to query row 0
 *   page list  = page_of[b][g][k_pos0/P .. (T_b-1)/P] (every id must be in
 *                [0, num_pages), else SEGKV_ERR_OUT_OF_RANGE; ids before
 *                k_pos0/P are not read and may be -1)
 *   k_len      = T_b - k_pos0
 *   pairs[s]   = G * sum over new rows i of |visible keys of i|   (int64)
 * Also emits cu_seqlens_q [S+1], cu_seqlens_k [num_segments+1] (prefix sums
 * of k_len), cu_pages [num_segments+1], and the attention kernel's work
 * list: every (segment, row block, head block) once, ordered by descending
 * cost (KV tiles visited) so that a launch dispatches the longest units
 * first (longest-processing-time-first balance across heads of very unequal
 * length). The order is by cost between consecutive windows of 512 units
 * only: inside a window the units are dealt so that positions x, x+8, x+16,
 * ... (the workgroups one XCD receives) hold neighbours in (segment, row)
 * order, which then share that XCD's L2.
 *
 * retain_lp [num_segments]: the first logical page a later query of the
 * segment can still see, so the caller may free the pages before it once
 * this step is done: 0 for a global head; floor(max(0, T_b - W + 1) / P) for
 * a local head (the next query, at position T_b, sees keys >= T_b - W + 1).
 *
 * Split-KV (page_size >= 64 only). With max_unit_tiles == 0 the builder splits
 * when the longest block would visit more than 3/4 of the mean tiles per
 * workgroup slot (512 slots): then every block longer than
 * max(16, ceil(mean / 2)) tiles is cut into equal runs of at most that many.
 * max_unit_tiles > 0 cuts every block longer than that; < 0 never splits.
 * A split block's runs become separate units with workspace slots, and one
 * merge entry per block. segkv_attn_prefill needs workspace_bytes =
 * SEGKV_WORKSPACE_BYTES(num_parts, unit_rows, unit_heads, head_dim) of device
 * workspace: the partial results, and for units of 256 pairs the work queues.
 */
typedef struct segkv_table_inputs {
    int32_t num_seqs;
    int32_t max_lp;
    const int32_t *cached_len;  /* [num_seqs] c_b >= 0 */
    const int32_t *new_len;     /* [num_seqs] n_b >= 1 */
    const int8_t *head_class;   /* [hkv] 1 = global, 0 = local (this layer) */
    const int32_t *window;      /* [hkv] W >= 1 for local heads; ignored for global */
    const int32_t *page_of;     /* [num_seqs][hkv][max_lp] (this layer) */
    int32_t max_unit_tiles;     /* split-KV policy: 0 automatic, > 0 longest run, < 0 never */
} segkv_table_inputs;

typedef struct segkv_tables {
    /* capacities of the caller's buffers, in elements (set by the caller) */
    int32_t seg_cap;            /* segments: >= num_seqs * hkv */
    int32_t seq_cap;            /* sequences: >= num_seqs */
    int64_t page_cap;           /* page_list entries */
    int32_t unit_cap;           /* work units */
    /* sizes written by the builder (also when it returns SEGKV_ERR_CAPACITY) */
    int32_t num_segments;
    int32_t num_units;
    int64_t num_page_entries;
    int64_t total_pairs;        /* sum of pairs[] */
    int32_t total_q_rows;       /* sum of n_b */
    int32_t unit_rows;          /* query rows per work unit */
    int32_t unit_heads;         /* query heads per work unit */
    /* caller-owned host buffers (may be NULL when the matching capacity is 0) */
    int32_t *seg_desc;          /* [seg_cap][SEGKV_SEG_FIELDS] */
    int32_t *cu_seqlens_q;      /* [seq_cap + 1] */
    int32_t *cu_seqlens_k;      /* [seg_cap + 1] */
    int32_t *cu_pages;          /* [seg_cap + 1] */
    int32_t *page_list;         /* [page_cap] */
    int64_t *pairs;             /* [seg_cap] */
    int32_t *work;              /* [unit_cap][SEGKV_UNIT_FIELDS] */
    /* split-KV (appended): capacity, sizes, buffer */
    int32_t merge_cap;          /* merge entries (set by the caller) */
    int32_t num_merges;
    int32_t num_parts;          /* workspace slots */
    int64_t workspace_bytes;    /* SEGKV_WORKSPACE_BYTES(num_parts, unit_rows, unit_heads, head_dim) */
    int32_t *merge;             /* [merge_cap][SEGKV_MERGE_FIELDS] */
    int32_t *retain_lp;         /* [seg_cap] (appended), or NULL to skip */
} segkv_tables;

int segkv_build_head_tables(const segkv_ctx *ctx, const segkv_table_inputs *in, segkv_tables *out);

/* Device copies of one layer's tables, as consumed by segkv_attn_prefill. */
typedef struct segkv_dev_tables {
    const int32_t *seg_desc;    /* device [num_segments][SEGKV_SEG_FIELDS] */
    const int32_t *page_list;   /* device [num_page_entries] */
    const int32_t *work;        /* device [num_units][SEGKV_UNIT_FIELDS] */
    int32_t num_segments;
    int32_t num_units;
    int64_t num_page_entries;
    int32_t total_q_rows;
    int32_t unit_rows;          /* must equal the builder's values for this context */
    int32_t unit_heads;
    const int32_t *merge;       /* device [num_merges][SEGKV_MERGE_FIELDS], or NULL if none */
    int32_t num_merges;
    int32_t num_parts;
} segkv_dev_tables;

/*
 * EXECUTE: fused variable-length causal prefill attention over every
 * segment's visible keys, for all query heads, in one launch.
 *   q   : device bf16 [total_q_rows][hq][head_dim]
 *   o   : device [total_q_rows][hq][head_dim], fp32 or bf16 per o_dtype
 *   lse : device fp32 [hq][total_q_rows] natural-log sum of exp of the scaled
 *         scores, or NULL
 *   softmax_scale : multiplies q.k; <= 0 selects 1/sqrt(head_dim)
 *   workspace : device memory of at least SEGKV_WORKSPACE_BYTES(t->num_parts,
 *               t->unit_rows, t->unit_heads, head_dim) bytes, the builder's
 *               workspace_bytes (caller-owned; may be NULL when that is 0).
 *               Its contents need no initialisation and are scratch
 *               afterwards; calls that share a workspace must not overlap.
 *               With units of 256 pairs, head_dim 128 and pages of at least
 *               64 keys, and more units than CUs, the kernel is persistent:
 *               one workgroup per CU taking units from per-XCD queues in the
 *               workspace, and from the other XCDs' queues once its own is
 *               empty.
 * For query row t of segment s and query head h of its group, position
 * i = q_pos0 + t:  O = sum_j softmax_j(scale * q.k_j) v_j over the visible
 * keys j of i, computed with bf16 inputs, fp32 accumulation and an online
 * (running-maximum) softmax. Every output row is written exactly once: by its
 * unit, or, for a split block, by the merge pass that combines the runs'
 * partial results (O = sum_r 2^(m_r - M) O_r / sum_r 2^(m_r - M) l_r, M the
 * largest running maximum), launched on the same stream right after.
 */
int segkv_attn_prefill(const segkv_ctx *ctx, const segkv_dev_tables *t, const void *q, void *o,
                       int32_t o_dtype, float *lse, float softmax_scale, void *workspace,
                       int64_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * segkv_attn_prefill with the split-KV workspace taken from scratch memory
 * the library itself holds, SEGKV_NOALLOC_SCRATCH_BYTES of device memory on
 * every GPU it runs on, kept until the process ends. Arguments, results and
 * errors are segkv_attn_prefill's otherwise; tables whose workspace exceeds
 * SEGKV_NOALLOC_SCRATCH_BYTES (SEGKV_WORKSPACE_BYTES(t->num_parts, ...)) are
 * refused with SEGKV_ERR_CAPACITY before anything runs. Calls no allocator.
 * All calls on one GPU share that GPU's scratch, which keeps the last call's
 * partial results (nothing in it needs clearing): calls that overlap on one
 * GPU (several streams or threads) race, so the caller serialises them. The
 * first call on a device, with that device current, looks up the scratch's
 * device address (SEGKV_ERR_HIP if that fails).
 */
#define SEGKV_NOALLOC_SCRATCH_BYTES (64LL << 20)
int segkv_attn_prefill_noalloc(const segkv_ctx *ctx, const segkv_dev_tables *t, const void *q, void *o,
                               int32_t o_dtype, float *lse, float softmax_scale, void *stream);

/*
 * Attention mass of the step's new tokens (RedKnot summary page, "Sparse
 * FFN": only the tokens with the highest attention scores run the dense
 * FFN; this is the score). Run after segkv_attn_prefill on the same tables
 * and inputs, with the LSE it wrote:
 *   mass[q_row0(b) + t] = sum over query heads h and query rows t' of
 *                         sequence b that see position c_b + t of
 *                         exp(scale * q[t', h] . k[c_b + t] - lse[h][t'])
 *   q    : device bf16 [total_q_rows][hq][head_dim] (as for the attention)
 *   lse  : device fp32 [hq][total_q_rows] from segkv_attn_prefill
 *   mass : device fp32 [total_q_rows], overwritten (cleared first, then
 *          accumulated with float atomics: the summation order varies)
 * Needs page_size >= 64 and prefill-shaped units (tables whose sequences all
 * bring more than 32 / G new rows, or any tables built for page_size < 64,
 * are refused with SEGKV_ERR_UNSUPPORTED); split units are fine. Cached
 * tokens (positions < c_b) get no mass.
 */
int segkv_attn_mass(const segkv_ctx *ctx, const segkv_dev_tables *t, const void *q, const float *lse,
                    float softmax_scale, float *mass, void *stream);

/*
 * Sparse FFN token selection (RedKnot summary page, "Sparse FFN": the
 * top-k tokens by attention score run the dense FFN, the rest the residual
 * identity). For each sequence b, picks min(keep[b], n_b, cu_keep[b+1] -
 * cu_keep[b]) of its rows cu_rows[b] .. cu_rows[b+1]-1 with the largest mass
 * (ties to the lower row; zero, negative and NaN masses rank as zero) and
 * writes their row indices in ascending order to rows_out[cu_keep[b] ...].
 *   mass     : device fp32 [total_rows] (segkv_attn_mass)
 *   cu_rows  : device int32 [num_seqs+1]; keep: device int32 [num_seqs];
 *   cu_keep  : device int32 [num_seqs+1], the output offsets
 *   rows_out : device int32 [cu_keep[num_seqs]]
 * A sequence whose row range leaves [0, total_rows) is skipped. The result is
 * unique (no order freedom), so it is reproducible bit for bit.
 */
int segkv_select_tokens(const segkv_ctx *ctx, const float *mass, const int32_t *cu_rows, const int32_t *keep,
                        const int32_t *cu_keep, int32_t num_seqs, int64_t total_rows, int32_t *rows_out,
                        void *stream);

/*
 * Sparse FFN of the chosen tokens (RedKnot summary page, "Sparse FFN"),
 * a SwiGLU block applied in place as a residual:
 *   h[m]          = bf16( silu(Wg x[r_m]) * (Wu x[r_m]) )   silu(g) = g / (1 + e^-g)
 *   x[r_m]        = bf16( x[r_m] + Wd h[m] )
 * for the chosen rows r_m = sel_rows[m], m < n_sel (distinct; rows outside
 * [0, x_rows) are skipped); every other row of x keeps its value (the
 * residual identity path).
 *   x      : device bf16 [x_rows][d_model], updated in place
 *   w_gate, w_up : device bf16 [d_ff][d_model];  w_down : device bf16 [d_model][d_ff]
 *   h      : device workspace, at least n_sel * d_ff * 2 bytes (bf16 [n_sel][d_ff])
 * Products accumulate in fp32 on bf16 MFMA. d_model and d_ff must be
 * multiples of 128 (SEGKV_ERR_UNSUPPORTED otherwise) and every operand under
 * 4 GiB.
 */
int segkv_sparse_ffn(const segkv_ctx *ctx, void *x, int64_t x_rows, int32_t d_model, int32_t d_ff,
                     const int32_t *sel_rows, int64_t n_sel, const void *w_gate, const void *w_up,
                     const void *w_down, void *h, int64_t h_bytes, void *stream);

/*
 * RoPE re-alignment of reused K pages (position-independent KV reuse; RedKnot
 * summary page, "Elastic Sparsity": recovery begins with RoPE position
 * alignment). entries: device int32 [n][4] = {page, slot0, nslots, delta}.
 * Slots slot0 .. slot0 + nslots - 1 (cut at the page end) of K page `page`
 * hold rows encoded with rotary angles at positions p; afterwards they hold
 * the rows encoded at p + delta. Rotary angles add, so each pair of
 * dimensions (i, i + D/2), i < D/2, is rotated by a = delta * theta_i with
 * theta_i = rope_base^(-2 i / D):
 *     x' = x cos a - y sin a,   y' = x sin a + y cos a
 * (pairing and base follow the rotate-half convention of the Llama family;
 * the pages fix neither). The angles are evaluated in fp64, the rotation in
 * fp32, the result rounded to bf16 (nearest even). V pages are position-free
 * and untouched. An entry whose page id is outside [0, num_pages) or whose
 * slot range is empty is skipped; entries that overlap race. rope_base > 1.
 */
int segkv_rope_realign(const segkv_ctx *ctx, const int32_t *entries, int64_t n, float rope_base, void *stream);

/*
 * Read pages back in a dense layout (tests, debugging):
 *   page_ids : device int32 [n]
 *   k_out, v_out : device bf16 [n][page_size][head_dim] each (V un-transposed)
 * An id outside [0, num_pages) yields zeros.
 */
int segkv_gather_pages(const segkv_ctx *ctx, const int32_t *page_ids, int64_t n,
                       void *k_out, void *v_out, void *stream);

/* Message of the last failing call on this thread ("" if none). */
const char *segkv_last_error(void);

/* Library version string. */
const char *segkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SEGKV_H */
