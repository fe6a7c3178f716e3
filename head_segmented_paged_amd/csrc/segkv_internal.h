// Internal declarations shared by the host C++ and the HIP translation units.
#pragma once

#include "segkv.h"

struct segkv_ctx {
    segkv_config cfg;
};

namespace segkv {

// Record a message for segkv_last_error() and return code.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Keys per KV tile of the attention kernel (one LDS stage).
constexpr int kKvTile = 64;
// Query rows handled by one wavefront (one 32-wide MFMA column block).
constexpr int kWaveRows = 32;
// Wavefronts per attention workgroup: four, or for the pipelined kernel
// (pages of at least one tile) on long contexts eight, whose waves all read the
// same K/V tiles, so each staged tile feeds twice the MFMAs. Either way a CU
// holds eight waves, two per SIMD. Eight-wave units start and finish a whole
// CU at once, which costs more than the shared staging saves when the units'
// K/V runs are short: they are used from a mean of wide_min_keys(head_dim)
// visible keys per query row (and KV head) of the layer. Head dim 128 runs its
// eight-wave-shaped units on the two-block kernel, whose per-unit start is
// cheaper, so it switches earlier.
constexpr int kWaves = 4;
constexpr int kWideWaves = 8;
inline int64_t wide_min_keys(int head_dim) { return head_dim == 128 ? 1024 : 2048; }
inline int unit_waves(int page_size, bool long_context)
{
    return page_size >= kKvTile && long_context ? kWideWaves : kWaves;
}
// Work-list cohorts: XCDs of the device (workgroups are dealt to them
// round-robin by index) and the workgroups one XCD holds at a time (32 CUs of
// eight waves each).
constexpr int kXcds = 8;
constexpr int kCuPerXcd = 32;
inline int cohort(int waves) { return kCuPerXcd * (2 * kWaves) / waves; }
// The same for decode work lists (single-wave workgroups, dealt like the
// four-wave ones).
constexpr int kCohort = 64;
// Shortest run the automatic split-KV policy cuts a block into (tiles).
constexpr int kMinRun = 16;

// Shape of one attention work unit for a given GQA group size G: the
// workgroup's `waves` wavefronts cover `heads` query heads of one group times
// `rows` query rows, one (head, 32-row block) per wavefront; `heads` is the
// largest power of two up to the wave count that divides G.
struct UnitShape {
    int rows;
    int heads;
};
inline UnitShape unit_shape(int G, int waves)
{
    int heads = 1;
    while (2 * heads <= waves && G % (2 * heads) == 0) heads *= 2;
    return UnitShape{kWaveRows * (waves / heads), heads};
}

// Decode / small-chunk units: every new row of a segment (at most 32 / G)
// for all G heads of its KV head, one (row, head) pair per MFMA column.
inline bool decode_units(int G, int page_size, int max_new_rows)
{
    return page_size >= kKvTile && G <= kWaveRows && max_new_rows <= kWaveRows / G;
}
inline UnitShape decode_shape(int G) { return UnitShape{kWaveRows / G, G}; }
// Workgroup slots of the decode kernel (eight single-wave workgroups per CU),
// the work units per slot its split-KV policy aims at, and the shortest run
// (in 64-key tiles) it cuts a block into.
constexpr int kDecodeSlots = 2048;
constexpr int kDecodeUnitsPerSlot = 1;
constexpr int kDecodeMinRun = 8;

inline bool supported_head_dim(int d) { return d == 64 || d == 128; }
inline bool supported_page_size(int p) { return p == 16 || p == 32 || p == 64 || p == 128 || p == 256; }

// Kernel launchers (segkv_kernels.hip). They assume validated arguments and
// return SEGKV_OK or SEGKV_ERR_HIP.
int launch_write_pages(const segkv_config &cfg, const void *k_new, const void *v_new, int64_t num_rows,
                       const int32_t *cu_rows, const int32_t *pos0, const int32_t *page_of, int32_t num_seqs,
                       int32_t max_lp, int32_t max_rows_per_seq, void *stream);
int launch_gather_pages(const segkv_config &cfg, const int32_t *page_ids, int64_t n, void *k_out, void *v_out,
                        void *stream);
int launch_rope_realign(const segkv_config &cfg, const int32_t *entries, int64_t n, float rope_base, void *stream);
int launch_select_tokens(const float *mass, const int32_t *cu_rows, const int32_t *keep, const int32_t *cu_keep,
                         int32_t num_seqs, int64_t total_rows, int32_t *rows_out, void *stream);
int launch_sparse_ffn(void *x, int64_t x_rows, int32_t d_model, int32_t d_ff, const int32_t *sel_rows,
                      int32_t n_sel, const void *w_gate, const void *w_up, const void *w_down, void *h, void *stream);
int launch_attn_mass(const segkv_config &cfg, const segkv_dev_tables &t, const void *q, const float *lse,
                     float scale_log2, float *mass, void *stream);
int launch_attn_prefill(const segkv_config &cfg, const segkv_dev_tables &t, const void *q, void *o,
                        int32_t o_dtype, float *lse, float scale_log2, void *workspace, void *stream);
// Device address of the library's no-alloc scratch on the current device
// (SEGKV_NOALLOC_SCRATCH_BYTES), looked up on the first call per device.
int noalloc_scratch(void **out);

}  // namespace segkv
