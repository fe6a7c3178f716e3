// C entry points: context, argument validation, error reporting, dispatch to
// the HIP launchers. Nothing here touches device memory.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <new>

#include "segkv_internal.h"

namespace segkv {

namespace {
thread_local char g_error[512] = "";
}

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_error[0] = '\0'; }

}  // namespace segkv

using segkv::fail;

extern "C" const char *segkv_last_error(void) { return segkv::g_error; }

extern "C" const char *segkv_version(void) { return "segkv 0.1 gfx950"; }

extern "C" int segkv_create(const segkv_config *cfg, segkv_ctx **out)
{
    segkv::clear_error();
    if (!cfg || !out) return fail(SEGKV_ERR_INVALID_ARG, "create: null argument");
    *out = nullptr;
    if (cfg->num_q_heads < 1 || cfg->num_kv_heads < 1 || cfg->num_q_heads % cfg->num_kv_heads != 0)
        return fail(SEGKV_ERR_INVALID_ARG, "create: num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                    cfg->num_q_heads, cfg->num_kv_heads);
    if (!segkv::supported_head_dim(cfg->head_dim))
        return fail(SEGKV_ERR_UNSUPPORTED, "create: head_dim %d not supported (64, 128)", cfg->head_dim);
    if (!segkv::supported_page_size(cfg->page_size))
        return fail(SEGKV_ERR_UNSUPPORTED, "create: page_size %d not supported (16, 32, 64, 128, 256)",
                    cfg->page_size);
    if (cfg->num_pages < 1 || cfg->num_pages > (int64_t{1} << 31) - 1)
        return fail(SEGKV_ERR_INVALID_ARG, "create: num_pages must be in [1, 2^31)");
    if (!cfg->k_pool || !cfg->v_pool) return fail(SEGKV_ERR_INVALID_ARG, "create: null pool pointer");
    segkv_ctx *ctx = new (std::nothrow) segkv_ctx;
    if (!ctx) return fail(SEGKV_ERR_INVALID_ARG, "create: out of host memory");
    ctx->cfg = *cfg;
    *out = ctx;
    return SEGKV_OK;
}

extern "C" void segkv_destroy(segkv_ctx *ctx) { delete ctx; }

extern "C" int segkv_write_pages(const segkv_ctx *ctx, const void *k_new, const void *v_new, int64_t num_rows,
                                 const int32_t *cu_rows, const int32_t *pos0, const int32_t *page_of,
                                 int32_t num_seqs, int32_t max_lp, int32_t max_rows_per_seq, void *stream)
{
    segkv::clear_error();
    if (!ctx) return fail(SEGKV_ERR_INVALID_ARG, "write_pages: null context");
    if (num_seqs < 1 || max_lp < 1 || max_rows_per_seq < 0 || num_rows < 0)
        return fail(SEGKV_ERR_INVALID_ARG, "write_pages: bad sizes (num_seqs %d, max_lp %d, max_rows %d)",
                    num_seqs, max_lp, max_rows_per_seq);
    if (num_rows == 0 || max_rows_per_seq == 0) return SEGKV_OK;
    if (!k_new || !v_new || !cu_rows || !pos0 || !page_of)
        return fail(SEGKV_ERR_INVALID_ARG, "write_pages: null pointer");
    return segkv::launch_write_pages(ctx->cfg, k_new, v_new, num_rows, cu_rows, pos0, page_of, num_seqs, max_lp,
                                     max_rows_per_seq, stream);
}

extern "C" int segkv_gather_pages(const segkv_ctx *ctx, const int32_t *page_ids, int64_t n, void *k_out,
                                  void *v_out, void *stream)
{
    segkv::clear_error();
    if (!ctx) return fail(SEGKV_ERR_INVALID_ARG, "gather_pages: null context");
    if (n < 0) return fail(SEGKV_ERR_INVALID_ARG, "gather_pages: negative count");
    if (n == 0) return SEGKV_OK;
    if (!page_ids || !k_out || !v_out) return fail(SEGKV_ERR_INVALID_ARG, "gather_pages: null pointer");
    return segkv::launch_gather_pages(ctx->cfg, page_ids, n, k_out, v_out, stream);
}

extern "C" int segkv_attn_mass(const segkv_ctx *ctx, const segkv_dev_tables *t, const void *q, const float *lse,
                               float softmax_scale, float *mass, void *stream)
{
    segkv::clear_error();
    if (!ctx || !t) return fail(SEGKV_ERR_INVALID_ARG, "attn_mass: null argument");
    const segkv_config &cfg = ctx->cfg;
    if (cfg.page_size < 64) return fail(SEGKV_ERR_UNSUPPORTED, "attn_mass: needs page_size >= 64");
    const int G = cfg.num_q_heads / cfg.num_kv_heads;
    const segkv::UnitShape s4 = segkv::unit_shape(G, segkv::kWaves), s8 = segkv::unit_shape(G, segkv::kWideWaves);
    if ((t->unit_rows != s4.rows || t->unit_heads != s4.heads) && (t->unit_rows != s8.rows || t->unit_heads != s8.heads))
        return fail(SEGKV_ERR_UNSUPPORTED, "attn_mass: needs prefill units of %d rows x %d heads or %d x %d (tables "
                    "have %d x %d)", s4.rows, s4.heads, s8.rows, s8.heads, t->unit_rows, t->unit_heads);
    if (t->num_segments < 0 || t->num_units < 0 || t->num_page_entries < 0 || t->total_q_rows < 0)
        return fail(SEGKV_ERR_INVALID_ARG, "attn_mass: negative table size");
    if (t->total_q_rows == 0) return SEGKV_OK;
    if (!mass || !lse || !q || (t->num_units > 0 && (!t->seg_desc || !t->page_list || !t->work)))
        return fail(SEGKV_ERR_INVALID_ARG, "attn_mass: null pointer");
    float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(static_cast<float>(cfg.head_dim));
    return segkv::launch_attn_mass(cfg, *t, q, lse, scale * 1.44269504088896340736f, mass, stream);
}

extern "C" int segkv_select_tokens(const segkv_ctx *ctx, const float *mass, const int32_t *cu_rows,
                                   const int32_t *keep, const int32_t *cu_keep, int32_t num_seqs,
                                   int64_t total_rows, int32_t *rows_out, void *stream)
{
    segkv::clear_error();
    if (!ctx) return fail(SEGKV_ERR_INVALID_ARG, "select_tokens: null context");
    if (num_seqs < 0 || total_rows < 0 || total_rows > 0x7fffffff)
        return fail(SEGKV_ERR_INVALID_ARG, "select_tokens: bad sizes");
    if (num_seqs == 0) return SEGKV_OK;
    if (!mass || !cu_rows || !keep || !cu_keep || !rows_out)
        return fail(SEGKV_ERR_INVALID_ARG, "select_tokens: null pointer");
    return segkv::launch_select_tokens(mass, cu_rows, keep, cu_keep, num_seqs, total_rows, rows_out, stream);
}

extern "C" int segkv_sparse_ffn(const segkv_ctx *ctx, void *x, int64_t x_rows, int32_t d_model, int32_t d_ff,
                                const int32_t *sel_rows, int64_t n_sel, const void *w_gate, const void *w_up,
                                const void *w_down, void *h, int64_t h_bytes, void *stream)
{
    segkv::clear_error();
    if (!ctx) return fail(SEGKV_ERR_INVALID_ARG, "sparse_ffn: null context");
    if (x_rows < 0 || n_sel < 0 || n_sel > 0x7fffffff || d_model < 1 || d_ff < 1)
        return fail(SEGKV_ERR_INVALID_ARG, "sparse_ffn: bad sizes");
    if (d_model % 128 != 0 || d_ff % 128 != 0)
        return fail(SEGKV_ERR_UNSUPPORTED, "sparse_ffn: d_model (%d) and d_ff (%d) must be multiples of 128",
                    d_model, d_ff);
    if (x_rows * d_model * 2 > 0xffffffffll || static_cast<int64_t>(d_ff) * d_model * 2 > 0xffffffffll ||
        n_sel * d_ff * 2 > 0xffffffffll)
        return fail(SEGKV_ERR_UNSUPPORTED, "sparse_ffn: an operand exceeds 4 GiB");
    if (n_sel == 0) return SEGKV_OK;
    if (!x || !sel_rows || !w_gate || !w_up || !w_down || !h)
        return fail(SEGKV_ERR_INVALID_ARG, "sparse_ffn: null pointer");
    if (h_bytes < n_sel * d_ff * 2)
        return fail(SEGKV_ERR_CAPACITY, "sparse_ffn: workspace h needs %lld bytes, %lld given",
                    static_cast<long long>(n_sel * d_ff * 2), static_cast<long long>(h_bytes));
    return segkv::launch_sparse_ffn(x, x_rows, d_model, d_ff, sel_rows, static_cast<int32_t>(n_sel), w_gate, w_up,
                                    w_down, h, stream);
}

extern "C" int segkv_rope_realign(const segkv_ctx *ctx, const int32_t *entries, int64_t n, float rope_base,
                                  void *stream)
{
    segkv::clear_error();
    if (!ctx) return fail(SEGKV_ERR_INVALID_ARG, "rope_realign: null context");
    if (n < 0 || n > 0x7fffffff) return fail(SEGKV_ERR_INVALID_ARG, "rope_realign: entry count out of range");
    if (!(rope_base > 1.0f) || !std::isfinite(rope_base))
        return fail(SEGKV_ERR_INVALID_ARG, "rope_realign: rope_base must be a finite value > 1");
    if (n == 0) return SEGKV_OK;
    if (!entries) return fail(SEGKV_ERR_INVALID_ARG, "rope_realign: null entries");
    return segkv::launch_rope_realign(ctx->cfg, entries, n, rope_base, stream);
}

namespace {

// segkv_attn_prefill; with noalloc the workspace is the library's scratch
// (workspace / workspace_bytes ignored).
int attn_prefill(const segkv_ctx *ctx, const segkv_dev_tables *t, const void *q, void *o, int32_t o_dtype,
                 float *lse, float softmax_scale, void *workspace, int64_t workspace_bytes, void *stream,
                 bool noalloc)
{
    segkv::clear_error();
    if (!ctx || !t) return fail(SEGKV_ERR_INVALID_ARG, "attn_prefill: null argument");
    const segkv_config &cfg = ctx->cfg;
    if (o_dtype != SEGKV_DTYPE_F32 && o_dtype != SEGKV_DTYPE_BF16)
        return fail(SEGKV_ERR_INVALID_ARG, "attn_prefill: o_dtype must be SEGKV_DTYPE_F32 or SEGKV_DTYPE_BF16");
    const int G = cfg.num_q_heads / cfg.num_kv_heads;
    const segkv::UnitShape shape = segkv::unit_shape(G, segkv::kWaves);
    const segkv::UnitShape wide = segkv::unit_shape(G, segkv::kWideWaves);
    const bool decode_ok = segkv::decode_units(G, cfg.page_size, 1) && t->unit_rows == segkv::decode_shape(G).rows &&
                           t->unit_heads == segkv::decode_shape(G).heads;
    const bool wide_ok = cfg.page_size >= segkv::kKvTile && t->unit_rows == wide.rows && t->unit_heads == wide.heads;
    if ((t->unit_rows != shape.rows || t->unit_heads != shape.heads) && !decode_ok && !wide_ok)
        return fail(SEGKV_ERR_INVALID_ARG, "attn_prefill: tables built for units of %d rows x %d heads, kernels "
                    "use %d x %d (with pages >= 64 also %d x %d, and %d x %d for decode)", t->unit_rows,
                    t->unit_heads, shape.rows, shape.heads, wide.rows, wide.heads, segkv::decode_shape(G).rows,
                    segkv::decode_shape(G).heads);
    if (t->num_segments < 0 || t->num_units < 0 || t->num_page_entries < 0 || t->total_q_rows < 0 ||
        t->num_merges < 0 || t->num_parts < 0)
        return fail(SEGKV_ERR_INVALID_ARG, "attn_prefill: negative table size");
    if (t->num_units == 0) return SEGKV_OK;
    if (!t->seg_desc || !t->page_list || !t->work || !q || !o)
        return fail(SEGKV_ERR_INVALID_ARG, "attn_prefill: null pointer");
    if (t->num_parts > 0 || t->num_merges > 0) {
        if (cfg.page_size < 64)
            return fail(SEGKV_ERR_UNSUPPORTED, "attn_prefill: split units need page_size >= 64");
        if (t->num_merges > 0 && !t->merge) return fail(SEGKV_ERR_INVALID_ARG, "attn_prefill: null merge list");
    }
    const int64_t need = SEGKV_WORKSPACE_BYTES(t->num_parts, t->unit_rows, t->unit_heads, cfg.head_dim);
    if (need > 0) {
        if (noalloc) {
            if (need > SEGKV_NOALLOC_SCRATCH_BYTES)
                return fail(SEGKV_ERR_CAPACITY, "attn_prefill_noalloc: workspace of %lld bytes needed, the "
                            "scratch holds %lld", static_cast<long long>(need),
                            static_cast<long long>(SEGKV_NOALLOC_SCRATCH_BYTES));
            const int rc = segkv::noalloc_scratch(&workspace);
            if (rc != SEGKV_OK) return rc;
        } else if (!workspace || workspace_bytes < need) {
            return fail(SEGKV_ERR_CAPACITY, "attn_prefill: workspace of %lld bytes needed, %lld given",
                        static_cast<long long>(need), static_cast<long long>(workspace ? workspace_bytes : 0));
        }
    }
    float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(static_cast<float>(cfg.head_dim));
    const float scale_log2 = scale * 1.44269504088896340736f;  // scores enter exp2 pre-multiplied by log2(e)
    return segkv::launch_attn_prefill(cfg, *t, q, o, o_dtype, lse, scale_log2, workspace, stream);
}

}  // namespace

extern "C" int segkv_attn_prefill(const segkv_ctx *ctx, const segkv_dev_tables *t, const void *q, void *o,
                                  int32_t o_dtype, float *lse, float softmax_scale, void *workspace,
                                  int64_t workspace_bytes, void *stream)
{
    return attn_prefill(ctx, t, q, o, o_dtype, lse, softmax_scale, workspace, workspace_bytes, stream, false);
}

extern "C" int segkv_attn_prefill_noalloc(const segkv_ctx *ctx, const segkv_dev_tables *t, const void *q, void *o,
                                          int32_t o_dtype, float *lse, float softmax_scale, void *stream)
{
    return attn_prefill(ctx, t, q, o, o_dtype, lse, softmax_scale, nullptr, 0, stream, true);
}
