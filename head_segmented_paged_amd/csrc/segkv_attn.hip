// Fused variable-length SegPaged prefill attention (EXECUTE) for gfx950.
//
// RedKnot summary page, "SegPaged Attention": one fused varlen pass over the
// per-(layer, KV head) page segments, with no attention-mask tensor; each
// head only reads the pages its visible keys live in. Global heads see the
// full causal context, local heads a sliding window ("Head-Class
// Sparsification"). The softmax is blockwise with a running maximum carried
// across KV blocks, the cross-block offset idea of the KV-cache management
// page (section 5.2), and the next KV block is fetched while the current one
// is being computed (same page, section 4.2).
//
// Work decomposition. One workgroup = one work unit from the host-built
// list (longest first): `rows` consecutive query rows of one segment for
// `heads` query heads of the segment's GQA group. Its four wavefronts each
// own one (query head, 32-row block); all of them consume the same K/V tiles
// from LDS, so a staged tile serves 128 query rows.
//
// Per KV tile of 64 keys, each wavefront computes on bf16 MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate):
//   S^T[key][query] = K . Q^T     A = K rows from LDS, B = Q^T held in VGPRs
//   O^T[d][query]  += V^T . P^T   A = V^T rows from LDS, B = P^T from S^T
// With S^T in the accumulator layout every lane holds one query column, so
// the row maximum and row sum are lane-local plus one exchange between the
// two 32-lane halves, and the rescale of O is a per-lane scalar. The K rows
// are fed to the S^T product in a swizzled order (bits 2 and 3 of the row
// index swapped) so that each lane's S^T accumulator registers, converted to
// bf16, are exactly the 8 consecutive keys the P^T operand of the next
// product needs; the V pages are stored key-innermost so the matching V^T
// operand is one 16-byte LDS read.
//
// Masking is index arithmetic on the tiles that cross the causal diagonal or
// the window edge; tiles inside a wavefront's band run unmasked. (The
// register-staged kernel for small pages skips tiles outside the band; the
// pipelined one computes them fully masked, which happens only at the band
// edges of units with several row blocks.) Keys outside the segment's
// stored-and-visible range are zero-filled in LDS so an undefined slot can
// never reach P.V.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "segkv_internal.h"

namespace segkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

constexpr int kBK = kKvTile;            // keys per tile
constexpr int kThreads = kWaves * 64;   // 256
constexpr float kRescaleSlack = 8.0f;   // log2-domain headroom before the running max is refreshed
constexpr float kNegBig = -1.0e30f;     // finite "no key yet" running max

template <int D>
struct Tile {
    static constexpr int kLd = D + 8;                 // K tile row stride (elements), 16-byte padded
    static constexpr int vLd = kBK + 8;               // V^T tile row stride (elements)
    static constexpr int kElems = kBK * kLd;
    static constexpr int vElems = D * vLd;
    static constexpr int stage = kElems + vElems;     // one LDS stage: K tile + V^T tile
    static constexpr int kPerThread = kBK * D / 8 / kThreads;   // 16-byte chunks per thread
    static constexpr int vPerThread = D * kBK / 8 / kThreads;
};

template <int D>
struct Staged {
    u32x4 k[Tile<D>::kPerThread];
    u32x4 v[Tile<D>::vPerThread];
    unsigned ok;  // bit r: K chunk r usable; bit 8 + r: V chunk r has a usable page
};

// K row fed to MFMA row r: bits 2 and 3 of r swapped.
__device__ __forceinline__ int swizzle_row(int r) { return (r & 0x13) | ((r & 4) << 1) | ((r & 8) >> 1); }

// NaN-propagating maximum (v_maximum3_f32 in chains): unlike fmaxf it needs no
// quieting of its operands.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Lanes l and l ^ 32 exchange x through v_permlane32_swap (upper half of the
// first operand <-> lower half of the second). The second operand is a copy
// the compiler cannot see through: with two operands it can prove equal it
// folds the swap's second result into the first.
__device__ __forceinline__ void swap_halves(float x, float &a, float &b)
{
    unsigned u = __builtin_bit_cast(unsigned, x), v = u;
    asm volatile("" : "+v"(v));
    const auto r = __builtin_amdgcn_permlane32_swap(u, v, false, false);
    a = __builtin_bit_cast(float, static_cast<unsigned>(r[0]));
    b = __builtin_bit_cast(float, static_cast<unsigned>(r[1]));
}

__device__ __forceinline__ float max_halves(float x)
{
    float a, b;
    swap_halves(x, a, b);
    return vmax(a, b);
}

__device__ __forceinline__ float sum_halves(float x)
{
    float a, b;
    swap_halves(x, a, b);
    return a + b;
}

// acc + the sum of the eight bf16 values in x, as four bf16 dot products with
// (1, 1): the softmax denominator then sums exactly the rounded probabilities
// that multiply V, in half the instructions of eight fp32 adds.
__device__ __forceinline__ float sum8_bf16(bf16x8 x, float acc)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), one, acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), one, acc, false);
}

// Physical page holding logical page lp of the segment, or -1.
__device__ __forceinline__ int page_id(const int32_t *__restrict__ pages, int n_pages, int64_t num_pages, int lp)
{
    const int id = pages[min(max(lp, 0), n_pages - 1)];
    return (lp >= 0 && lp < n_pages && id >= 0 && id < num_pages) ? id : -1;
}

// Issue the loads of one KV tile (keys tile_key0 .. tile_key0+63 of the
// segment) into registers. The tile spans 64 / P pages: each lane looks up
// its chunks' page ids first (all id loads together), then issues its data
// loads from valid addresses; whether a chunk may be used is recorded in
// st.ok and applied when the tile is written to LDS, so the loads of a tile
// are all in flight together and nothing waits on them here.
template <int D>
__device__ __forceinline__ void fetch_tile(Staged<D> &st, const u16 *__restrict__ kpool,
                                           const u16 *__restrict__ vpool, const int32_t *__restrict__ pages,
                                           int32_t n_pages, int64_t num_pages, int log2P, int tile_key0, int zero_lo,
                                           int zero_hi)
{
    const int pmask = (1 << log2P) - 1;
    int kpage[Tile<D>::kPerThread], vpage[Tile<D>::vPerThread];
#pragma unroll
    for (int r = 0; r < Tile<D>::kPerThread; ++r) {
        const int c = threadIdx.x + r * kThreads;
        kpage[r] = page_id(pages, n_pages, num_pages, (tile_key0 + c / (D / 8)) >> log2P);
    }
#pragma unroll
    for (int r = 0; r < Tile<D>::vPerThread; ++r) {
        const int c = threadIdx.x + r * kThreads;
        vpage[r] = page_id(pages, n_pages, num_pages, (tile_key0 + (c % (kBK / 8)) * 8) >> log2P);
    }
    unsigned ok = 0;
#pragma unroll
    for (int r = 0; r < Tile<D>::kPerThread; ++r) {
        const int c = threadIdx.x + r * kThreads;
        const int key = c / (D / 8), dc = c % (D / 8);
        const int idx = tile_key0 + key;
        const bool use = idx >= zero_lo && idx < zero_hi && kpage[r] >= 0;
        const int64_t pg = use ? kpage[r] : 0;
        ok |= use ? (1u << r) : 0u;
        st.k[r] = *reinterpret_cast<const u32x4 *>(kpool + ((pg << log2P) + (idx & pmask)) * D + dc * 8);
    }
#pragma unroll
    for (int r = 0; r < Tile<D>::vPerThread; ++r) {
        const int c = threadIdx.x + r * kThreads;
        const int d = c / (kBK / 8), kc = c % (kBK / 8);
        const int idx0 = tile_key0 + kc * 8;
        const bool use = idx0 + 7 >= zero_lo && idx0 < zero_hi && vpage[r] >= 0;
        const int64_t pg = use ? vpage[r] : 0;
        ok |= use ? (1u << (8 + r)) : 0u;
        st.v[r] = *reinterpret_cast<const u32x4 *>(vpool + ((pg * D + d) << log2P) + (idx0 & pmask));
    }
    st.ok = ok;
}

// Write a fetched tile to one LDS stage, zeroing what must not be used
// (keys outside [zero_lo, zero_hi) or on a missing page).
template <int D>
__device__ __forceinline__ void store_tile(const Staged<D> &st, u16 *__restrict__ stage, int tile_key0,
                                           int zero_lo, int zero_hi)
{
    u16 *ks = stage;
    u16 *vs = stage + Tile<D>::kElems;
#pragma unroll
    for (int r = 0; r < Tile<D>::kPerThread; ++r) {
        const int c = threadIdx.x + r * kThreads;
        const int key = c / (D / 8), dc = c % (D / 8);
        const u32x4 z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4 *>(ks + key * Tile<D>::kLd + dc * 8) = (st.ok >> r) & 1u ? st.k[r] : z;
    }
#pragma unroll
    for (int r = 0; r < Tile<D>::vPerThread; ++r) {
        const int c = threadIdx.x + r * kThreads;
        const int d = c / (kBK / 8), kc = c % (kBK / 8);
        const int idx0 = tile_key0 + kc * 8;
        u32x4 val = (st.ok >> (8 + r)) & 1u ? st.v[r] : u32x4{0u, 0u, 0u, 0u};
        if (idx0 < zero_lo || idx0 + 8 > zero_hi) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int idx = idx0 + i;
                if (idx < zero_lo || idx >= zero_hi) val[i >> 1] &= (i & 1) ? 0x0000ffffu : 0xffff0000u;
            }
        }
        *reinterpret_cast<u32x4 *>(vs + d * Tile<D>::vLd + kc * 8) = val;
    }
}

// Register-staged kernel for pages shorter than a tile (16 or 32 keys): a
// tile spans several pages, so each lane fetches its chunks into registers
// and writes them to a padded LDS stage, with no cross-tile pipeline.
template <int D, int HPW, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 2) void attn_prefill_kernel(
    const u16 *__restrict__ q, const u16 *__restrict__ kpool, const u16 *__restrict__ vpool, int64_t num_pages,
    int log2P, const int32_t *__restrict__ seg_desc, const int32_t *__restrict__ page_list,
    int64_t num_page_entries, const int32_t *__restrict__ work, int32_t num_segments, int32_t total_q_rows,
    int32_t hq, float scale_log2, void *__restrict__ o, float *__restrict__ lse)
{
    using T = Tile<D>;
    constexpr int kRowBlocks = kWaves / HPW;
    constexpr int kUnitRows = kWaveRows * kRowBlocks;
    constexpr int kSteps = D / 16;      // MFMA k-steps over the head dim for S^T
    constexpr int kDBlocks = D / 32;    // 32-row blocks of O^T
    __shared__ __attribute__((aligned(16))) u16 smem[2 * T::stage];

    const i32x4 unit = *reinterpret_cast<const i32x4 *>(work + static_cast<int64_t>(blockIdx.x) * SEGKV_UNIT_FIELDS);
    const int seg = unit[SEGKV_UNIT_SEGMENT], row0 = unit[SEGKV_UNIT_ROW0], head0 = unit[SEGKV_UNIT_HEAD0];
    if (seg < 0 || seg >= num_segments) return;
    const int32_t *desc = seg_desc + static_cast<int64_t>(seg) * SEGKV_SEG_FIELDS;
    const int q_row0 = desc[SEGKV_SEG_Q_ROW0], n_q = desc[SEGKV_SEG_N_Q], q_pos0 = desc[SEGKV_SEG_Q_POS0];
    const int window = desc[SEGKV_SEG_WINDOW], k_pos0 = desc[SEGKV_SEG_K_POS0], k_len = desc[SEGKV_SEG_K_LEN];
    const int page_off = desc[SEGKV_SEG_PAGE_OFF];
    if (row0 < 0 || row0 >= n_q || page_off < 0 || page_off >= num_page_entries || k_len < 1) return;
    int n_pages = (k_len + (1 << log2P) - 1) >> log2P;
    if (n_pages > num_page_entries - page_off) n_pages = static_cast<int>(num_page_entries - page_off);
    const int32_t *pages = page_list + page_off;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const int head = head0 + wave % HPW;
    const int wrow0 = row0 + (wave / HPW) * kWaveRows;

    // Key band of the whole unit, as tile indices relative to k_pos0.
    const int unit_end = min(row0 + kUnitRows, n_q);
    const int first_pos = q_pos0 + row0, last_pos = q_pos0 + unit_end - 1;
    const int lo_pos = window ? max(0, first_pos - window + 1) : 0;
    const int tile_beg = (lo_pos - k_pos0) / kBK;
    const int tile_end = (last_pos + 1 - k_pos0 + kBK - 1) / kBK;
    // Stored keys that some query of the segment can see; everything else is zero-filled.
    const int zero_lo = max(0, (window ? max(0, q_pos0 - window + 1) : 0) - k_pos0);
    const int zero_hi = k_len;

    // This wavefront's rows.
    const bool wave_valid = wrow0 < n_q && head < hq;
    const int wrow_end = min(wrow0 + kWaveRows, n_q);
    const int wp_lo = q_pos0 + wrow0, wp_hi = q_pos0 + wrow_end - 1;
    const int my_t = min(wrow0 + col, n_q - 1);
    const int my_pos = q_pos0 + my_t;
    const int lo_i = window ? my_pos - window + 1 : -(1 << 30);   // first visible key position of this lane's row
    const int64_t my_row = static_cast<int64_t>(q_row0) + my_t;
    const bool row_ok = wave_valid && (wrow0 + col) < n_q && my_row < total_q_rows;

    bf16x8 qreg[kSteps];
    {
        const bool can_load = wave_valid && my_row < total_q_rows;
        const u16 *qp = q + (my_row * hq + head) * D + 8 * half;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (can_load) raw = *reinterpret_cast<const u32x4 *>(qp + 16 * s);
            qreg[s] = __builtin_bit_cast(bf16x8, raw);
        }
    }

    f32x16 oacc[kDBlocks];
#pragma unroll
    for (int i = 0; i < kDBlocks; ++i) oacc[i] = f32x16{};
    float m = kNegBig, lsum = 0.f;

    // Tile jt covers keys [64 jt, 64 jt + 64) of the segment.
    auto fetch = [&](Staged<D> &st, int jt) {
        fetch_tile<D>(st, kpool, vpool, pages, n_pages, num_pages, log2P, jt * kBK, zero_lo, zero_hi);
    };
    auto store = [&](const Staged<D> &st, u16 *stage, int jt) { store_tile<D>(st, stage, jt * kBK, zero_lo, zero_hi); };
    Staged<D> st;
    fetch(st, tile_beg);
    store(st, smem, tile_beg);
    __syncthreads();

    for (int jt = tile_beg; jt < tile_end; ++jt) {
        const int cur = (jt - tile_beg) & 1;
        const bool more = jt + 1 < tile_end;
        if (more) fetch(st, jt + 1);

        const u16 *ks = smem + cur * T::stage;
        const u16 *vs = ks + T::kElems;
        const int kp0 = k_pos0 + jt * kBK;
        const bool active = wave_valid && kp0 <= wp_hi && !(window && kp0 + kBK - 1 < wp_lo - window + 1);
        if (active) {
            const bool full = (kp0 + kBK - 1 <= wp_lo) && (window == 0 || kp0 >= wp_hi - window + 1);
            // S^T = K . Q^T, two 32-key blocks.
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                sacc[kb] = f32x16{};
                const u16 *krow = ks + (32 * kb + swizzle_row(col)) * T::kLd + 8 * half;
#pragma unroll
                for (int s = 0; s < kSteps; ++s) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(krow + 16 * s);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], sacc[kb], 0, 0, 0);
                }
            }
            if (!full) {
                // key position of accumulator element e of block kb = kbase + const;
                // visible iff lo_i <= position <= my_pos, one unsigned range test each
                const int kbase = kp0 + 8 * half;
                const unsigned span = static_cast<unsigned>(my_pos - lo_i);
                const int off = kbase - lo_i;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int jj = e >> 2, ii = e & 3;
                        const int kc = 32 * kb + 16 * (jj >> 1) + 4 * (jj & 1) + ii;
                        const bool vis = static_cast<unsigned>(off + kc) <= span;
                        sacc[kb][e] = vis ? sacc[kb][e] : -__builtin_inff();
                    }
            }
            // Running maximum (log2 domain), refreshed only when it grows by more than the slack.
            float mt = sacc[0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) mt = vmax(mt, sacc[kb][e]);
            mt = max_halves(mt) * scale_log2;
            if (__any(mt > m + kRescaleSlack)) {
                const float m_new = fmaxf(m, mt);
                const float alpha = __builtin_amdgcn_exp2f(m - m_new);
                lsum *= alpha;
#pragma unroll
                for (int i = 0; i < kDBlocks; ++i) oacc[i] *= alpha;
                m = m_new;
            }
            // P = exp2(S * scale * log2(e) - m), packed to bf16 B operands and summed per lane.
            bf16x8 pb[4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][e], scale_log2, -m));
                    pb[2 * kb + (e >> 3)][e & 7] = static_cast<__bf16>(p);
                }
            lsum += sum8_bf16(pb[0], 0.f) + sum8_bf16(pb[1], 0.f) + sum8_bf16(pb[2], 0.f) + sum8_bf16(pb[3], 0.f);
            // O^T += V^T . P^T, four 16-key steps.
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db) {
                const u16 *vrow = vs + (32 * db + col) * T::vLd + 8 * half;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vrow + 16 * t);
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[t], oacc[db], 0, 0, 0);
                }
            }
        }
        if (more) store(st, smem + (cur ^ 1) * T::stage, jt + 1);
        __syncthreads();
    }

    // Epilogue: combine the two halves' row sums, normalise, store.
    const float ltot = sum_halves(lsum);
    if (!row_ok) return;
    const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
    const int64_t obase = (my_row * hq + head) * D;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int d0 = 32 * db + 8 * jj + 4 * half;
            const float v0 = oacc[db][4 * jj + 0] * inv, v1 = oacc[db][4 * jj + 1] * inv;
            const float v2 = oacc[db][4 * jj + 2] * inv, v3 = oacc[db][4 * jj + 3] * inv;
            if constexpr (OUT_BF16) {
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                bf16x4 w = {static_cast<__bf16>(v0), static_cast<__bf16>(v1), static_cast<__bf16>(v2),
                            static_cast<__bf16>(v3)};
                *reinterpret_cast<bf16x4 *>(static_cast<u16 *>(o) + obase + d0) = w;
            } else {
                typedef float f32x4 __attribute__((ext_vector_type(4)));
                *reinterpret_cast<f32x4 *>(static_cast<float *>(o) + obase + d0) = f32x4{v0, v1, v2, v3};
            }
        }
    if (lse && half == 0)
        lse[static_cast<int64_t>(head) * total_q_rows + my_row] = (m + __log2f(ltot)) * 0.69314718055994530942f;
}

// ---------------------------------------------------------------------------
// Page size >= 64. A KV tile then lies inside one page, and its K and V^T
// rows are copied straight from the pools into LDS by the load unit
// (global_load_lds_dwordx4: each lane's 16 bytes land at M0 + 16 * lane),
// so no VGPRs hold a tile in flight and those registers go to a deeper LDS
// operand prefetch instead. Because a DMA writes 1 KiB contiguously per
// wave instruction, tile rows are unpadded; an XOR swizzle of the 16-byte
// chunk position keeps the MFMA operand reads free of bank conflicts. The
// two LDS stages are separate arrays so the compiler can see that reading
// one never waits for the DMA into the other.
template <int D, int NW>
struct DmaTile {
    static constexpr int kRowBytes = D * 2;                   // one key of K
    static constexpr int kBytes = kBK * kRowBytes;            // K tile
    static constexpr int vBytes = D * kBK * 2;                // V^T tile: D rows of 64 keys
    static constexpr int bytes = kBytes + vBytes;
    static constexpr int kInstr = kBytes / 1024 / NW;         // DMA instructions per wave
    static constexpr int vInstr = vBytes / 1024 / NW;
    static_assert(kInstr >= 1 && vInstr >= 1, "each wave moves at least one KB of a tile");
};
// Chunk swizzles: K row r keeps logical chunk c at position c ^ kswz(r); V^T
// row d keeps key chunk c at position c ^ vswz(d).
template <int D>
__device__ __forceinline__ int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
__device__ __forceinline__ int vswz(int d) { return (d >> 1) & 7; }

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from a buffer resource straight into LDS at lds + 16 * lane.
// (A device function: the builtin must not appear in the kernel body itself,
// where the host pass would drop the kernel's launch stub.)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, char *lds, unsigned voffset, unsigned soffset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)lds, 16, voffset, soffset, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const u16 *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<u16 *>(base), 0, bytes, 0x00020000);
}

// Software-pipelined kernel for pages of at least one tile (K and V tiles
// DMA'd straight from the page into LDS, XOR-swizzled). K runs one tile
// ahead of V: while a wavefront turns tile j's scores into probabilities and
// accumulates P(j) V(j), it already issues the MFMAs for tile j+1's scores, so
// the matrix cores have independent work during the softmax arithmetic.
// Buffers: K(j+1) and V(j) are read while K(j+2) and V(j+1) land, two K and two
// V tiles (the same 64 KB as two whole stages for D = 128).
template <int D, int HPW, bool OUT_BF16, int NW>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attn_prefill_pipe_kernel(
    const u16 *__restrict__ q, const u16 *__restrict__ kpool, const u16 *__restrict__ vpool, int64_t num_pages,
    int log2P, const int32_t *__restrict__ seg_desc, const int32_t *__restrict__ page_list,
    int64_t num_page_entries, const int32_t *__restrict__ work, int32_t num_segments, int32_t total_q_rows,
    int32_t hq, float scale_log2, void *__restrict__ o, float *__restrict__ lse, float *__restrict__ parts,
    int32_t num_parts)
{
    using T = DmaTile<D, NW>;
    constexpr int kRowBlocks = NW / HPW;
    constexpr int kUnitRows = kWaveRows * kRowBlocks;
    constexpr int kSteps = D / 16;      // MFMA k-steps over the head dim for S^T
    constexpr int kDBlocks = D / 32;    // 32-row blocks of O^T
    // Separate arrays, so the compiler sees that a DMA into one buffer does not
    // alias the LDS reads of another and adds no wait for it.
    __shared__ __attribute__((aligned(1024))) char kbuf0[T::kBytes];
    __shared__ __attribute__((aligned(1024))) char kbuf1[T::kBytes];
    __shared__ __attribute__((aligned(1024))) char vbuf0[T::vBytes];
    __shared__ __attribute__((aligned(1024))) char vbuf1[T::vBytes];

    const int32_t *urec = work + static_cast<int64_t>(blockIdx.x) * SEGKV_UNIT_FIELDS;
    const i32x4 unit = *reinterpret_cast<const i32x4 *>(urec);
    const i32x4 unit2 = *reinterpret_cast<const i32x4 *>(urec + 4);
    const int seg = unit[SEGKV_UNIT_SEGMENT], row0 = unit[SEGKV_UNIT_ROW0], head0 = unit[SEGKV_UNIT_HEAD0];
    const int run0 = unit2[SEGKV_UNIT_TILE0 - 4], run_len = unit[SEGKV_UNIT_TILES];
    const int part = unit2[SEGKV_UNIT_PART - 4];
    if (seg < 0 || seg >= num_segments || part >= num_parts) return;
    const int32_t *desc = seg_desc + static_cast<int64_t>(seg) * SEGKV_SEG_FIELDS;
    const int q_row0 = desc[SEGKV_SEG_Q_ROW0], n_q = desc[SEGKV_SEG_N_Q], q_pos0 = desc[SEGKV_SEG_Q_POS0];
    const int window = desc[SEGKV_SEG_WINDOW], k_pos0 = desc[SEGKV_SEG_K_POS0], k_len = desc[SEGKV_SEG_K_LEN];
    const int page_off = desc[SEGKV_SEG_PAGE_OFF];
    if (row0 < 0 || row0 >= n_q || page_off < 0 || page_off >= num_page_entries || k_len < 1) return;
    int n_pages = (k_len + (1 << log2P) - 1) >> log2P;
    if (n_pages > num_page_entries - page_off) n_pages = static_cast<int>(num_page_entries - page_off);
    const int32_t *pages = page_list + page_off;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const int head = head0 + wave % HPW;
    const int wrow0 = row0 + (wave / HPW) * kWaveRows;

    const int unit_end = min(row0 + kUnitRows, n_q);
    const int first_pos = q_pos0 + row0, last_pos = q_pos0 + unit_end - 1;
    const int lo_pos = window ? max(0, first_pos - window + 1) : 0;
    // The unit's run of tiles, within the band its rows see.
    const int tile_beg = max((lo_pos - k_pos0) / kBK, run0);
    const int tile_end = min((last_pos + 1 - k_pos0 + kBK - 1) / kBK, run0 + max(run_len, 0));
    const int zero_lo = max(0, (window ? max(0, q_pos0 - window + 1) : 0) - k_pos0);
    const int zero_hi = k_len;

    const bool wave_valid = wrow0 < n_q && head < hq;
    const int wrow_end = min(wrow0 + kWaveRows, n_q);
    const int wp_lo = q_pos0 + wrow0, wp_hi = q_pos0 + wrow_end - 1;
    const int my_t = min(wrow0 + col, n_q - 1);
    const int my_pos = q_pos0 + my_t;
    const int lo_i = window ? my_pos - window + 1 : -(1 << 30);
    const int64_t my_row = static_cast<int64_t>(q_row0) + my_t;
    const bool row_ok = wave_valid && (wrow0 + col) < n_q && my_row < total_q_rows;

    bf16x8 qreg[kSteps];
    {
        const bool can_load = wave_valid && my_row < total_q_rows;
        const u16 *qp = q + (my_row * hq + head) * D + 8 * half;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (can_load) raw = *reinterpret_cast<const u32x4 *>(qp + 16 * s);
            qreg[s] = __builtin_bit_cast(bf16x8, raw);
        }
    }
    f32x16 oacc[kDBlocks];
#pragma unroll
    for (int i = 0; i < kDBlocks; ++i) oacc[i] = f32x16{};
    float m = kNegBig, lsum = 0.f;

    // Page ids: a 64-entry register window per wave, read with v_readlane.
    // Lookups must come in non-decreasing tile order, at most one window apart.
    int win = ((tile_beg * kBK) >> log2P) >> 6;
    auto load_window = [&](int w) { return pages[min(w * 64 + lane, n_pages - 1)]; };
    int win_cur = load_window(win), win_next = load_window(win + 1);
    auto tile_page = [&](int jt) {
        const int lp = (jt * kBK) >> log2P;
        if ((lp >> 6) != win) {
            win = lp >> 6;
            win_cur = win_next;
            win_next = load_window(win + 1);
        }
        const int id = __builtin_amdgcn_readlane(win_cur, lp & 63);
        return (lp < n_pages && id >= 0 && id < num_pages) ? id : -1;
    };

    // Per-lane DMA source offsets (bytes from the tile's first key in its page).
    unsigned kdma[T::kInstr], vdma[T::vInstr];
#pragma unroll
    for (int i = 0; i < T::kInstr; ++i) {
        const int p = (wave * T::kInstr + i) * 1024 + lane * 16;
        const int r = p / T::kRowBytes, c = ((p % T::kRowBytes) / 16) ^ kswz<D>(r);
        kdma[i] = static_cast<unsigned>(r * T::kRowBytes + c * 16);
    }
#pragma unroll
    for (int i = 0; i < T::vInstr; ++i) {
        const int p = (wave * T::vInstr + i) * 1024 + lane * 16;
        const int d = p / 128, c = ((p % 128) / 16) ^ vswz(d);
        vdma[i] = static_cast<unsigned>(((d << log2P) + c * 8) * 2);
    }
    // One buffer resource per page: an out-of-range offset, or a missing page
    // (zero records), reads as zeros.
    auto dma_k = [&](char *dst, int page, int jt) {
        const unsigned slot0 = static_cast<unsigned>((jt * kBK) & ((1 << log2P) - 1));
        const int64_t pg = page >= 0 ? page : 0;
        const __amdgpu_buffer_rsrc_t rk =
            page_rsrc(kpool + ((pg * D) << log2P), page >= 0 ? (T::kRowBytes << log2P) : 0);
#pragma unroll
        for (int i = 0; i < T::kInstr; ++i)
            dma16(rk, dst + (wave * T::kInstr + i) * 1024, kdma[i], slot0 * T::kRowBytes);
    };
    auto dma_v = [&](char *dst, int page, int jt) {
        const unsigned slot0 = static_cast<unsigned>((jt * kBK) & ((1 << log2P) - 1));
        const int64_t pg = page >= 0 ? page : 0;
        const __amdgpu_buffer_rsrc_t rv = page_rsrc(vpool + ((pg * D) << log2P), page >= 0 ? ((D * 2) << log2P) : 0);
#pragma unroll
        for (int i = 0; i < T::vInstr; ++i)
            dma16(rv, dst + (wave * T::vInstr + i) * 1024, vdma[i], slot0 * 2);
    };
    // A tile that holds keys outside [zero_lo, zero_hi) gets those V^T entries
    // zeroed once it has landed (their scores are masked, but 0 * NaN would
    // still reach the accumulator).
    auto edge_tile = [&](int jt) {
        const int key0 = jt * kBK;
        return key0 < zero_lo || key0 + kBK > zero_hi;
    };
    auto fixup = [&](char *vb, int jt) {
        const int key0 = jt * kBK;
        for (int e = threadIdx.x; e < D * kBK; e += NW * 64) {
            const int d = e / kBK, k = e % kBK, idx = key0 + k;
            if (idx < zero_lo || idx >= zero_hi)
                *reinterpret_cast<u16 *>(vb + d * 128 + (((k >> 3) ^ vswz(d)) << 4) + (k & 7) * 2) = 0;
        }
    };

    // Per-lane LDS operand addresses within a K tile and a V^T tile.
    const int krow = swizzle_row(col);
    unsigned ka[kSteps], va[4];
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
        ka[s] = static_cast<unsigned>(krow * T::kRowBytes + (((2 * s + half) ^ kswz<D>(krow)) << 4));
#pragma unroll
    for (int t = 0; t < 4; ++t) va[t] = static_cast<unsigned>(col * 128 + (((2 * t + half) ^ vswz(col)) << 4));

    auto tile_full = [&](int jt) {
        const int kp0 = k_pos0 + jt * kBK;
        return (kp0 + kBK - 1 <= wp_lo) && (window == 0 || kp0 >= wp_hi - window + 1);
    };

    // S^T k-step s of the next tile: two 32-key MFMAs.
    auto score_step = [&](f32x16 (&sn)[2], const char *kb, int s) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kb + ka[s] + h * 32 * T::kRowBytes);
            sn[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], s == 0 ? f32x16{} : sn[h], 0, 0, 0);
        }
    };
    // First k-steps of the next tile's scores go out before the masking and
    // rescale branches; the rest are spread over the four probability chunks.
    constexpr int kEarly = 2;
    auto step_lo = [](int t) { return kEarly + (t * (kSteps - kEarly)) / 4; };

    // One tile: scores sc of tile jt (already computed) -> P -> O^T += V^T P^T;
    // when NEXT, the scores of tile jt + 1 from kn into sn on the side.
    auto tile = [&](auto next, int jt, const char *kn, const char *vc, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
        constexpr bool NEXT = decltype(next)::value;
        if constexpr (NEXT) {
#pragma unroll
            for (int s = 0; s < kEarly; ++s) score_step(sn, kn, s);
        }
        if (!tile_full(jt)) {
            const int kbase = k_pos0 + jt * kBK + 8 * half;
            const unsigned span = static_cast<unsigned>(my_pos - lo_i);
            const int off = kbase - lo_i;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int jj = e >> 2, ii = e & 3;
                    const int kc = 32 * h + 16 * (jj >> 1) + 4 * (jj & 1) + ii;
                    sc[h][e] = static_cast<unsigned>(off + kc) <= span ? sc[h][e] : -__builtin_inff();
                }
        }
        // Tile max: four independent chains of three-operand maxima. The
        // NaN-propagating maximum needs no quieting of the MFMA results
        // (v_maximum3_f32); a NaN score would reach O through P either way.
        float mx[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int e0 = 8 * (c & 1);
            mx[c] = vmax(sc[c >> 1][e0], sc[c >> 1][e0 + 1]);
#pragma unroll
            for (int e = 2; e < 8; e += 2) mx[c] = vmax(vmax(mx[c], sc[c >> 1][e0 + e]), sc[c >> 1][e0 + e + 1]);
        }
        float mt = vmax(vmax(mx[0], mx[1]), vmax(mx[2], mx[3]));
        mt = max_halves(mt) * scale_log2;
        if (__any(mt > m + kRescaleSlack)) {
            const float m_new = fmaxf(m, mt);
            const float alpha = __builtin_amdgcn_exp2f(m - m_new);
            lsum *= alpha;
#pragma unroll
            for (int i = 0; i < kDBlocks; ++i) oacc[i] *= alpha;
            m = m_new;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bf16x8 pb;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                pb[i] = static_cast<__bf16>(
                    __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t >> 1][8 * (t & 1) + i], scale_log2, -m)));
            lsum = sum8_bf16(pb, lsum);
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vc + va[t] + db * 32 * 128);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[db], 0, 0, 0);
            }
            if constexpr (NEXT) {
#pragma unroll
                for (int s = step_lo(t); s < step_lo(t + 1); ++s) score_step(sn, kn, s);
            }
        }
        if constexpr (NEXT) {
            // Operands read four MFMAs ahead; about four VALU ops beside each MFMA.
            constexpr int kMfma = 4 * kDBlocks + 2 * (kSteps - kEarly);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < kMfma - 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
        }
    };

    // Iteration jt: DMA V(jt+1) into vd and K(jt+2) into kd, compute tile jt
    // (and the scores of jt+1 when it exists), then wait for the DMA.
    int page_v = -1;   // page of tile jt+1, looked up when its K was fetched
    auto iteration = [&](auto next, int jt, char *kn, char *vc, char *kd, char *vd, f32x16 (&sc)[2],
                         f32x16 (&sn)[2]) {
        constexpr bool NEXT = decltype(next)::value;
        if constexpr (NEXT) {
            dma_v(vd, page_v, jt + 1);
            if (jt + 2 < tile_end) {
                page_v = tile_page(jt + 2);
                dma_k(kd, page_v, jt + 2);
            }
        }
        tile(next, jt, kn, vc, sc, sn);
        if constexpr (NEXT) {
            __syncthreads();
            if (edge_tile(jt + 1)) {
                fixup(vd, jt + 1);
                __syncthreads();
            }
        }
    };

    f32x16 sa[2], sb[2];
    if (tile_beg < tile_end) {
        const int page0 = tile_page(tile_beg);
        dma_k(kbuf0, page0, tile_beg);
        dma_v(vbuf0, page0, tile_beg);
        if (tile_beg + 1 < tile_end) {
            page_v = tile_page(tile_beg + 1);
            dma_k(kbuf1, page_v, tile_beg + 1);
        }
        __syncthreads();
        if (edge_tile(tile_beg)) fixup(vbuf0, tile_beg);
#pragma unroll
        for (int s = 0; s < kSteps; ++s) score_step(sa, kbuf0, s);
        __syncthreads();   // kbuf0 is refilled by the first iteration
    }
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;
    if (tile_beg < tile_end) {
        int jt = tile_beg;
        for (; jt + 2 < tile_end; jt += 2) {
            iteration(yes{}, jt, kbuf1, vbuf0, kbuf0, vbuf1, sa, sb);
            iteration(yes{}, jt + 1, kbuf0, vbuf1, kbuf1, vbuf0, sb, sa);
        }
        if (jt + 1 < tile_end) {
            iteration(yes{}, jt, kbuf1, vbuf0, kbuf0, vbuf1, sa, sb);
            iteration(no{}, jt + 1, kbuf0, vbuf1, kbuf1, vbuf0, sb, sa);
        } else {
            iteration(no{}, jt, kbuf1, vbuf0, kbuf0, vbuf1, sa, sb);
        }
    }

    const float ltot = sum_halves(lsum);
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    // Lane (col, half) holds O^T dims 32 db + 8 jj + 4 half + i of its row as
    // oacc[db][4 jj + i]. Stored from there, each store instruction would put
    // 16 or 32 bytes into each of 32 rows (32 cache lines). Where the two K
    // buffers hold 8 KB per wave (head dim 128, four waves) the rows leave
    // through them instead: the last tile reads only its V^T buffer, and its
    // K buffer was last read before the previous iteration's barrier. Row r
    // of the wave is staged at r * 256 bytes, its 16-byte chunk c at chunk
    // position c ^ (r & 15) (the 32 rows of one write instruction spread over
    // the banks), all 128 dims in bf16 or 64 of them per pass in fp32, and
    // stored whole: 1 KB contiguous per store instruction within a row.
    constexpr int kStageWave = 8192;
    constexpr bool kStaged = D == 128 && NW == 4 && T::kBytes == 2 * kStageWave;
    auto put_rows = [&](auto f32_c, float sc, char *dst0, int64_t stride, int nrows) {
        constexpr bool F32 = decltype(f32_c)::value;
        constexpr int EB = F32 ? 4 : 2, RB = 256, CH = RB / 16, RPP = 1024 / RB, NP = kWaveRows / RPP;
        constexpr int DBP = RB / (32 * EB);   // dim blocks per pass
        char *const stage = (wave < NW / 2 ? kbuf0 : kbuf1) + (wave % (NW / 2)) * kStageWave;
        const int rl = lane / CH, c = lane % CH;
#pragma unroll
        for (int p = 0; p < kDBlocks / DBP; ++p) {
            asm volatile("" ::: "memory");   // after the previous pass's reads
#pragma unroll
            for (int dbl = 0; dbl < DBP; ++dbl)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int db = p * DBP + dbl;
                    const int b0 = (32 * dbl + 8 * jj + 4 * half) * EB;   // byte offset within the row
                    char *pp = stage + col * RB + (((b0 >> 4) ^ (col & 15)) << 4) + (b0 & 15);
                    const float x0 = oacc[db][4 * jj] * sc, x1 = oacc[db][4 * jj + 1] * sc;
                    const float x2 = oacc[db][4 * jj + 2] * sc, x3 = oacc[db][4 * jj + 3] * sc;
                    if constexpr (F32)
                        *reinterpret_cast<f32x4 *>(pp) = f32x4{x0, x1, x2, x3};
                    else
                        *reinterpret_cast<bf16x4 *>(pp) = bf16x4{static_cast<__bf16>(x0), static_cast<__bf16>(x1),
                                                                 static_cast<__bf16>(x2), static_cast<__bf16>(x3)};
                }
            // lanes read rows other lanes wrote: one wavefront's LDS
            // operations complete in order; only the compiler must keep them so
            asm volatile("" ::: "memory");
            char *g = dst0 + rl * stride + p * RB + 16 * c;
#pragma unroll
            for (int p0 = 0; p0 < NP; p0 += 4) {
                u32x4 x[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = (p0 + i) * RPP + rl;
                    x[i] = *reinterpret_cast<const u32x4 *>(stage + rr * RB + ((c ^ (rr & 15)) << 4));
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if ((p0 + i) * RPP + rl < nrows) *reinterpret_cast<u32x4 *>(g + (p0 + i) * RPP * stride) = x[i];
            }
        }
    };
    if (part >= 0) {
        // Split unit: unnormalised O, running maximum and sum to its slot:
        // [pairs][D] outputs, then [pairs] maxima, then [pairs] sums, pair
        // r = (head offset) * unit rows + (row offset).
        constexpr int kPairs = kUnitRows * HPW;   // (row, head) pairs per unit
        float *slot = parts + static_cast<int64_t>(part) * (kPairs * (D + 2));
        const int r0 = (wave % HPW) * kUnitRows + (wave / HPW) * kWaveRows;   // the wave's first slot row
        const int r = r0 + col;
        if constexpr (kStaged) {
            put_rows(std::true_type{}, 1.0f, reinterpret_cast<char *>(slot + static_cast<int64_t>(r0) * D), D * 4,
                     kWaveRows);
        } else {
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    *reinterpret_cast<f32x4 *>(slot + r * D + 32 * db + 8 * jj + 4 * half) =
                        f32x4{oacc[db][4 * jj], oacc[db][4 * jj + 1], oacc[db][4 * jj + 2], oacc[db][4 * jj + 3]};
        }
        if (half == 0) {
            slot[kPairs * D + r] = m;
            slot[kPairs * (D + 1) + r] = ltot;
        }
        return;
    }
    const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
    if constexpr (kStaged) {
        constexpr int EB = OUT_BF16 ? 2 : 4;
        const int64_t grow0 = static_cast<int64_t>(q_row0) + wrow0;   // the wave's first row of O
        const int nrows = wave_valid ? static_cast<int>(min<int64_t>(n_q - wrow0, total_q_rows - grow0)) : 0;
        put_rows(std::integral_constant<bool, !OUT_BF16>{}, inv,
                 static_cast<char *>(o) + (grow0 * hq + head) * D * EB, static_cast<int64_t>(hq) * D * EB, nrows);
    } else if (row_ok) {
        const int64_t obase = (my_row * hq + head) * D;
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d0 = 32 * db + 8 * jj + 4 * half;
                const float v0 = oacc[db][4 * jj + 0] * inv, v1 = oacc[db][4 * jj + 1] * inv;
                const float v2 = oacc[db][4 * jj + 2] * inv, v3 = oacc[db][4 * jj + 3] * inv;
                if constexpr (OUT_BF16) {
                    *reinterpret_cast<bf16x4 *>(static_cast<u16 *>(o) + obase + d0) =
                        bf16x4{static_cast<__bf16>(v0), static_cast<__bf16>(v1), static_cast<__bf16>(v2),
                               static_cast<__bf16>(v3)};
                } else {
                    *reinterpret_cast<f32x4 *>(static_cast<float *>(o) + obase + d0) = f32x4{v0, v1, v2, v3};
                }
            }
    }
    if (lse && half == 0 && row_ok)
        lse[static_cast<int64_t>(head) * total_q_rows + my_row] = (m + __log2f(ltot)) * 0.69314718055994530942f;
}

// ---------------------------------------------------------------------------
// Two-block prefill kernel (head dim 128, pages of at least one tile, units
// of 256 (row, head) pairs). One wavefront per SIMD, each owning two
// 32-column query blocks, so every K and V^T operand read from LDS feeds two
// MFMAs: half the LDS operand traffic per FLOP of the one-block kernels,
// whose two waves per SIMD each read their own copy of every operand (the
// CU's LDS bandwidth, not the matrix cores, bounded those). The price is the
// register state of 64 query columns: O^T (128 registers) and Q^T (64) live
// in AGPRs as the MFMA accumulator and B operand, the scores of two tiles
// (128) in VGPRs. That state is held in registers the compiler may not
// allocate (the kernel's own code is limited to 64 VGPRs and 64 AGPRs) and
// is touched only by the generated blocks of segkv_tile_asm.inc (written by
// gen_tile_asm.py), which issue one tile's scores-of-the-next-tile, softmax
// and P.V work in a fixed interleave. The loop around them (page ids, K/V
// DMA into LDS, barriers, masking decisions) is the pipelined kernel's, with
// four waves.
// Dynamic LDS of the two-block kernel: a three-slot ring of K tiles, a
// three-slot ring of V^T tiles, and the rows of Q on their way to the AGPRs.
constexpr unsigned kW2Slot = 16384;
constexpr unsigned kW2VRing = 3 * kW2Slot;
constexpr unsigned kW2Q = 6 * kW2Slot;          // Q staging rows, 16 KB per wave
constexpr unsigned kW2QWave = 16384;
constexpr unsigned kW2Lds = kW2Q + 4 * kW2QWave;

struct W2Addr {
    unsigned ka[8];          // K operand of k-step s: LDS byte offset within a K slot (lane's row and chunk)
    unsigned va[4];          // V^T operand of 16-key step t: LDS address within V slot 0
    unsigned kd[4], vd[4];   // the lane's DMA source offsets within a K / V page (bytes), less 1024 i
};
// Per-tile scalars of the tile bodies (wave-uniform).
struct W2Step {
    __amdgpu_buffer_rsrc_t rk, rv;   // source pages of the K tile three ahead and the V^T tile two ahead
    unsigned sok, sov;               // their first key's byte offset within the page
    unsigned m0k, m0v;               // LDS destination of this wave's DMA instructions
    unsigned kslot, vslot;           // LDS address of the K slot read now, offset of the V^T slot read now
};
// Scalars of a steady-state run (w2_run), fixed for the unit.
struct W2Run {
    unsigned kbase;                  // LDS address of the rings
    unsigned m0k, m0v;               // this wave's DMA destination in K slot 0 / V^T slot 0
    const int32_t *pages;            // the segment's page list
    unsigned kplo, kphi;             // K pool address
    unsigned vdlo, vdhi;             // V^T pool address minus K pool address (mod 2^64)
    unsigned pbytes;                 // bytes of one page of K (and of V^T)
    int64_t npg;                     // pages in the pool (ids outside [0, npg) are not pages)
    unsigned lastlp;                 // the segment's last page-list index
    unsigned log2p, pmask;           // log2 of the page size, page size - 1
};
// Masking of a tile's scores (lane-varying bounds, wave-uniform skip flag).
struct W2Mask {
    int a0, a1;                      // lo_i - tile start - 8 half, per block
    unsigned s0, s1;                 // pos_i - lo_i, per block
    unsigned full;                   // every key of the tile visible to every row of the wave
};

// The blocks clobber registers above the kernel's own budget on purpose (that
// is where their state lives), which clang reports for every block.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
#include "segkv_tile_asm.inc"
#pragma clang diagnostic pop

template <int HPW, bool OUT_BF16>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_num_vgpr(64))) void attn_prefill_w2_kernel(
    const u16 *__restrict__ q, const u16 *__restrict__ kpool, const u16 *__restrict__ vpool, int64_t num_pages,
    int log2P, const int32_t *__restrict__ seg_desc, const int32_t *__restrict__ page_list,
    int64_t num_page_entries, const int32_t *__restrict__ work, int32_t num_units, int32_t *__restrict__ queue,
    int32_t num_segments, int32_t total_q_rows, int32_t hq, float scale_log2, void *__restrict__ o,
    float *__restrict__ lse, float *__restrict__ parts, int32_t num_parts)
{
    constexpr int D = 128, NW = 4;
    using T = DmaTile<D, NW>;
    constexpr int kUnitRows = 256 / HPW;       // rows per unit (eight 32-row blocks over HPW heads)
    static_assert(T::kBytes == kW2Slot && T::vBytes == kW2Slot, "tile bodies assume 16 KB tiles");
    // kW2Lds bytes of dynamic LDS: the K ring, the V^T ring and the Q rows.
    // The LDS is dynamic so that the compiler's occupancy estimate does not
    // raise the kernel's own register budget into the range the tile bodies
    // keep their state in.
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    // Persistent workgroups (when there are more units than CUs; else one
    // unit each, queue null): workgroup w starts on unit w and then takes
    // units from the queue of its XCD (workgroups go to the XCDs round-robin
    // by index, and the table builder deals units so that those an XCD
    // receives are neighbours: queue x holds the units at or past the grid
    // whose index is x mod 8, in order), and once that queue is empty from
    // the other XCDs' queues. The XCDs' clocks differ by up to ~10 % under
    // this load, so a fixed share of units per XCD left the fast ones idle
    // at the end of the launch. Wave 0 requests the next unit as the current
    // one starts and passes it to the other waves through LDS (a word of its
    // Q staging rows, free once it has read its Q) at the barrier after the
    // first scores.
    const int xq = static_cast<int>(blockIdx.x % kXcds);
    int *const next_word = reinterpret_cast<int *>(smem + kW2Q);
    // One lane's fetch-and-add on a queue counter. The offset is one the
    // compiler cannot prove uniform: for a uniform address it would turn the
    // atomic into a wave-level one and read its result at once, waiting for
    // it there instead of where the result is used.
    auto fetch_add = [&](int32_t *counter) {
        int z;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z));
        return atomicAdd(counter + z, 1);
    };
    auto steal = [&]() -> int {   // the other XCDs' queues (only at the end of the launch)
        for (int i = 1; i < kXcds; ++i) {
            const int y = xq + i < kXcds ? xq + i : xq + i - kXcds;
            const int v = static_cast<int>(gridDim.x) + y + kXcds * fetch_add(queue + y);
            if (v < num_units) return v;
        }
        return num_units;
    };
    int u = static_cast<int>(blockIdx.x);
    for (;;) {
    int nxt = num_units;   // the workgroup's next unit
    // Per-unit copies the compiler cannot see through, so that nothing below
    // is computed once before the unit loop and then held (spilled) through
    // every unit.
    int lane_u = threadIdx.x & 63, wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int log2P_u = log2P, hq_u = hq;
    const u16 *q_u = q, *kpool_u = kpool, *vpool_u = vpool;
    asm volatile("" : "+v"(lane_u), "+s"(wave_u), "+s"(log2P_u), "+s"(hq_u), "+s"(q_u), "+s"(kpool_u),
                 "+s"(vpool_u));
    {
    const int log2P = log2P_u, hq = hq_u;
    const u16 *const q = q_u, *const kpool = kpool_u, *const vpool = vpool_u;
    const int wave = wave_u, lane = lane_u;
    // This unit's request on the XCD's queue (wave 0, lane 0): issued once the
    // unit's first transfers have landed (a vector-memory operation issued
    // before them would hold up their counted wait), read when the next
    // unit is published.
    int claim_t = 0;
    auto request = [&]() {
        if (queue && wave == 0 && lane == 0) claim_t = fetch_add(queue + xq);
    };
    // The next unit into next_word (wave 0, lane 0).
    auto publish = [&]() {
        if (wave == 0 && lane == 0) {
            int v = num_units;
            if (queue) {
                v = static_cast<int>(gridDim.x) + xq + kXcds * claim_t;
                if (v >= num_units) v = steal();
            }
            next_word[0] = v;
        }
    };

    const int32_t *urec = work + static_cast<int64_t>(u) * SEGKV_UNIT_FIELDS;
    const i32x4 unit = *reinterpret_cast<const i32x4 *>(urec);
    const i32x4 unit2 = *reinterpret_cast<const i32x4 *>(urec + 4);
    const i32x4 unit3 = *reinterpret_cast<const i32x4 *>(urec + 8);
    const int seg = unit[SEGKV_UNIT_SEGMENT], row0 = unit[SEGKV_UNIT_ROW0], head0 = unit[SEGKV_UNIT_HEAD0];
    const int run0 = unit2[SEGKV_UNIT_TILE0 - 4], run_len = unit[SEGKV_UNIT_TILES];
    const int part = unit2[SEGKV_UNIT_PART - 4];
    const bool seg_ok = seg >= 0 && seg < num_segments && part < num_parts;
    int q_row0 = 0, n_q = 0, q_pos0 = 0, window = 0, k_pos0 = 0, k_len = 0, page_off = 0;
    if (seg_ok) {
        const int32_t *desc = seg_desc + static_cast<int64_t>(seg) * SEGKV_SEG_FIELDS;
        q_row0 = desc[SEGKV_SEG_Q_ROW0], n_q = desc[SEGKV_SEG_N_Q], q_pos0 = desc[SEGKV_SEG_Q_POS0];
        window = desc[SEGKV_SEG_WINDOW], k_pos0 = desc[SEGKV_SEG_K_POS0], k_len = desc[SEGKV_SEG_K_LEN];
        page_off = desc[SEGKV_SEG_PAGE_OFF];
    }
    if (!seg_ok || row0 < 0 || row0 >= n_q || page_off < 0 || page_off >= num_page_entries || k_len < 1) {
        // a record that fails its checks (none the table builder writes): skipped
        request();
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        publish();
        __syncthreads();
        nxt = __builtin_amdgcn_readfirstlane(next_word[0]);
        __syncthreads();   // read by every wave before wave 0's next Q rows overwrite it
    } else {
    int n_pages = (k_len + (1 << log2P) - 1) >> log2P;
    if (n_pages > num_page_entries - page_off) n_pages = static_cast<int>(num_page_entries - page_off);
    const int32_t *pages = page_list + page_off;

    const int col = lane & 31, half = lane >> 5;
    // The wave's two blocks: consecutive 32-row blocks of one head, or (eight
    // heads per unit) one 32-row block of two heads.
    int hoff[2], rblk[2];
    if constexpr (HPW == 8) {
        hoff[0] = 2 * wave, hoff[1] = 2 * wave + 1, rblk[0] = rblk[1] = 0;
    } else {
        hoff[0] = hoff[1] = wave % HPW;
        rblk[0] = 2 * (wave / HPW), rblk[1] = 2 * (wave / HPW) + 1;
    }

    const int unit_end = min(row0 + kUnitRows, n_q);
    const int first_pos = q_pos0 + row0, last_pos = q_pos0 + unit_end - 1;
    const int lo_pos = window ? max(0, first_pos - window + 1) : 0;
    const int tile_beg = max((lo_pos - k_pos0) / kBK, run0);
    const int tile_end = min((last_pos + 1 - k_pos0 + kBK - 1) / kBK, run0 + max(run_len, 0));
    const int zero_lo = max(0, (window ? max(0, q_pos0 - window + 1) : 0) - k_pos0);
    const int zero_hi = k_len;

    // Page id of tile jt (or -1) from the segment's page list. Inside the
    // unit loop the compiler makes this a vector load and waits for it at
    // once (every DMA in flight with it); read through a constant-address
    // pointer it becomes a scalar load, which measured slower still: the
    // tile body then issued meanwhile counts it in its LDS waits. Only the
    // bodies outside the steady-state runs (a unit's edges) load ids here;
    // the runs read theirs in their own code. The index is clamped so the
    // load needs no branch; the id is checked when its buffer resource is
    // built.
    auto page_at = [&](int jt) {
        const int lp = __builtin_amdgcn_readfirstlane((jt * kBK) >> log2P);
        const int id = __builtin_amdgcn_readfirstlane(pages[min(max(lp, 0), n_pages - 1)]);
        return lp < 0 || lp >= n_pages ? -1 : id;
    };
    // Pages of tiles jt .. jt+3 at the top of the tile loop. The unit's first
    // four come with its work record when the record's run starts at the
    // unit's first visible tile (every unit the table builder makes), so the
    // first K/V transfers wait for no page-list read; else from the list.
    int pg[4];
    if (tile_beg == run0) {
        pg[0] = unit2[SEGKV_UNIT_PAGE0 - 4];
        pg[1] = tile_beg + 1 < tile_end ? unit2[SEGKV_UNIT_PAGE0 + 1 - 4] : -1;
        pg[2] = tile_beg + 2 < tile_end ? unit3[SEGKV_UNIT_PAGE0 + 2 - 8] : -1;
        pg[3] = tile_beg + 3 < tile_end ? unit3[SEGKV_UNIT_PAGE0 + 3 - 8] : -1;
    } else {
        pg[0] = page_at(tile_beg);
        pg[1] = tile_beg + 1 < tile_end ? page_at(tile_beg + 1) : -1;
        pg[2] = tile_beg + 2 < tile_end ? page_at(tile_beg + 2) : -1;
        pg[3] = tile_beg + 3 < tile_end ? page_at(tile_beg + 3) : -1;
    }

    // Per block: rows, positions, and whether the block exists.
    int wrow0[2], my_pos[2], lo_i[2], head[2];
    int64_t my_row[2];
    bool blk_ok[2], row_ok[2];
    int wr_first = 1 << 30, wr_last = -1;   // the wave's valid rows (relative to the segment)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        head[k] = head0 + hoff[k];
        wrow0[k] = row0 + rblk[k] * kWaveRows;
        blk_ok[k] = wrow0[k] < n_q && head[k] < hq;
        const int my_t = min(wrow0[k] + col, n_q - 1);
        my_pos[k] = q_pos0 + my_t;
        lo_i[k] = window ? my_pos[k] - window + 1 : -(1 << 30);
        my_row[k] = static_cast<int64_t>(q_row0) + my_t;
        row_ok[k] = blk_ok[k] && (wrow0[k] + col) < n_q && my_row[k] < total_q_rows;
        if (blk_ok[k]) {
            wr_first = min(wr_first, wrow0[k]);
            wr_last = max(wr_last, min(wrow0[k] + kWaveRows, n_q) - 1);
        }
    }
    const int wp_lo = q_pos0 + wr_first, wp_hi = q_pos0 + wr_last;

    const unsigned lds0 = static_cast<unsigned>(reinterpret_cast<uintptr_t>(smem));
    W2Addr ad;
#pragma unroll
    for (int i = 0; i < T::kInstr; ++i) {
        const int p = (wave * T::kInstr + i) * 1024 + lane * 16;
        const int rr = p / T::kRowBytes, c = ((p % T::kRowBytes) / 16) ^ kswz<D>(rr);
        ad.kd[i] = static_cast<unsigned>(rr * T::kRowBytes + c * 16 - 1024 * i);
    }
#pragma unroll
    for (int i = 0; i < T::vInstr; ++i) {
        const int p = (wave * T::vInstr + i) * 1024 + lane * 16;
        const int d = p / 128, c = ((p % 128) / 16) ^ vswz(d);
        ad.vd[i] = static_cast<unsigned>(((d << log2P) + c * 8) * 2 - 1024 * i);
    }
    {
        const int krow = swizzle_row(col);
#pragma unroll
        for (int s = 0; s < 8; ++s)
            ad.ka[s] = static_cast<unsigned>(krow * T::kRowBytes + (((2 * s + half) ^ kswz<D>(krow)) << 4));
#pragma unroll
        for (int t = 0; t < 4; ++t)
            ad.va[t] = lds0 + kW2VRing + static_cast<unsigned>(col * 128 + (((2 * t + half) ^ vswz(col)) << 4));
    }
    // Buffer resource of a tile's page (a missing page, or a tile past the
    // unit's run, has no records: its DMA reads zeros) and the byte offset of
    // the tile's first key in that page.
    auto k_rsrc = [&](int page) {
        const bool ok = page >= 0 && page < num_pages;
        const int64_t pg = ok ? page : 0;
        return page_rsrc(kpool + ((pg * D) << log2P), ok ? (T::kRowBytes << log2P) : 0);
    };
    auto v_rsrc = [&](int page) {
        const bool ok = page >= 0 && page < num_pages;
        const int64_t pg = ok ? page : 0;
        return page_rsrc(vpool + ((pg * D) << log2P), ok ? ((D * 2) << log2P) : 0);
    };
    auto slot0 = [&](int jt) { return static_cast<unsigned>((jt * kBK) & ((1 << log2P) - 1)); };
    auto dma_k = [&](unsigned slot, int page, int jt) {
        const __amdgpu_buffer_rsrc_t rk = k_rsrc(page);
#pragma unroll
        for (int i = 0; i < T::kInstr; ++i)
            dma16(rk, smem + slot * kW2Slot + (wave * T::kInstr + i) * 1024, ad.kd[i] + 1024 * i,
                  slot0(jt) * T::kRowBytes);
    };
    auto dma_v = [&](unsigned slot, int page, int jt) {
        const __amdgpu_buffer_rsrc_t rv = v_rsrc(page);
#pragma unroll
        for (int i = 0; i < T::vInstr; ++i)
            dma16(rv, smem + kW2VRing + slot * kW2Slot + (wave * T::vInstr + i) * 1024, ad.vd[i] + 1024 * i,
                  slot0(jt) * 2);
    };
    // Q of both blocks into the wave's LDS staging rows (issued now, waited
    // for before the first scores), whole rows per transfer: staging row r =
    // 32 qb + column holds that query's 256 bytes, 16-byte chunk c at chunk
    // position c ^ (r & 15), so each 1 KB transfer reads four rows whole (8
    // cache lines) where loads straight into the MFMA operand layout would
    // touch 32 rows per instruction. A buffer over the unit's rows of Q: a
    // lane whose row or head does not exist reads zeros.
    char *const qstage = smem + kW2Q + wave * kW2QWave;
    {
        const int64_t urow0 = static_cast<int64_t>(q_row0) + row0;   // first Q row of the unit
        const int64_t urows = max<int64_t>(0, min<int64_t>(unit_end - row0, total_q_rows - urow0));
        const __amdgpu_buffer_rsrc_t rq =
            page_rsrc(q + urow0 * hq * D, static_cast<int>(urows * hq * D * 2));
        const int rsub = lane >> 4, pos = lane & 15;   // row within the transfer's four, chunk position
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int k = i >> 3, cc = 4 * (i & 7) + rsub;   // block, column of staging row 4 i + rsub
            const int64_t row = static_cast<int64_t>(q_row0) + min(wrow0[k] + cc, n_q - 1);
            const bool can_load = blk_ok[k] && row < total_q_rows;
            const int c = pos ^ (cc & 15);
            dma16(rq, qstage + i * 1024,
                  can_load ? static_cast<unsigned>(((row - urow0) * hq + head[k]) * D * 2 + c * 16) : 0x80000000u, 0);
        }
    }
    // Then the unit's first K/V tiles (Q comes from memory, while the K/V
    // tiles are mostly still in the L2 from the neighbouring units' reads):
    // Q and these are what the first tile's scores wait for.
    if (tile_beg < tile_end) {
        dma_k(0, pg[0], tile_beg);
        dma_v(0, pg[0], tile_beg);
        dma_k(1, pg[1], tile_beg + 1);
        dma_v(1, pg[1], tile_beg + 1);
        dma_k(2, pg[2], tile_beg + 2);
    }
    w2_zero_o();
    float m0 = kNegBig, m1 = kNegBig, l0 = 0.f, l1 = 0.f;   // running maximum (log2 domain) and sum per block


    auto edge_tile = [&](int jt) {
        const int key0 = jt * kBK;
        return key0 < zero_lo || key0 + kBK > zero_hi;
    };
    auto fixup = [&](unsigned slot, int jt) {
        char *vb = smem + kW2VRing + slot * kW2Slot;
        const int key0 = jt * kBK;
        for (int e = threadIdx.x; e < D * kBK; e += NW * 64) {
            const int d = e / kBK, k = e % kBK, idx = key0 + k;
            if (idx < zero_lo || idx >= zero_hi)
                *reinterpret_cast<u16 *>(vb + d * 128 + (((k >> 3) ^ vswz(d)) << 4) + (k & 7) * 2) = 0;
        }
    };
    auto tile_full = [&](int jt) {
        const int kp0 = k_pos0 + jt * kBK;
        return (kp0 + kBK - 1 <= wp_lo) && (window == 0 || kp0 >= wp_hi - window + 1);
    };
    // Mask operands of tile jt: visible iff (key - lo_i) <= (pos - lo_i), unsigned.
    auto mask_args = [&](int jt, int k, int &a, unsigned &s) {
        const int kbase = k_pos0 + jt * kBK + 8 * half;
        a = lo_i[k] - kbase;
        s = static_cast<unsigned>(my_pos[k] - lo_i[k]);
    };
    auto mask = [&](int jt) {
        W2Mask mk;
        mask_args(jt, 0, mk.a0, mk.s0);
        mask_args(jt, 1, mk.a1, mk.s1);
        mk.full = __builtin_amdgcn_readfirstlane(tile_full(jt) ? 1u : 0u);
        return mk;
    };

    // Ring: tile jt's K tile sits in K slot (jt - tile_beg) % 3 and its V^T
    // tile in V slot (jt - tile_beg) % 3. The body of tile jt reads K(jt+1)
    // and V(jt), and issues the DMA of K(jt+3) and V(jt+2), whose slots held
    // K(jt) and V(jt-1), read by the previous body (before its barrier).
    if (tile_beg < tile_end) {
        // Q, K(0) and V(0) have landed for every wave (the transfers of K(1),
        // V(1) and K(2), issued after them, may still be in flight: the
        // counter counts down in issue order).
        constexpr int kAfterV0 = 2 * T::kInstr + T::vInstr;
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kAfterV0) : "memory");
        __builtin_amdgcn_s_barrier();
        request();
        if (edge_tile(tile_beg)) fixup(0, tile_beg);   // V(jt+1) is fixed after body jt's barrier
        {
            // Q^T from the staging rows (this wave's transfers, landed): k-step
            // s of block 0 for lane (col, half) is chunk 2 s + half of row col
            unsigned qa[8];
            const unsigned qrow = static_cast<unsigned>(reinterpret_cast<uintptr_t>(qstage)) + col * 256;
#pragma unroll
            for (int st = 0; st < 8; ++st) qa[st] = qrow + (((2 * st + half) ^ (col & 15)) << 4);
            w2_q_from_lds(qa);
        }
        W2Step st;
        st.kslot = lds0;
        st.vslot = 0;
        w2_scores_first(m0, m1, l0, l1, ad, st, mask(tile_beg), scale_log2);
        publish();         // wave 0 has read its Q rows, where the word lies
        __syncthreads();   // K slot 0 is refilled by the first body; the fixups are visible
        nxt = __builtin_amdgcn_readfirstlane(next_word[0]);
        unsigned sk = 0;   // K slot of tile jt (= slot of tile jt+3); V slot of jt is sk as well
        auto step = [&](int jt) {
            // scalars of the body of tile jt; the page of tile jt+4 is loaded
            // now and used a body later
            const unsigned sk1 = sk == 2 ? 0 : sk + 1, sk2 = sk1 == 2 ? 0 : sk1 + 1;
            const int pk = pg[3];
            W2Step s;
            s.rk = k_rsrc(pk);
            s.rv = v_rsrc(pg[2]);
            s.sok = slot0(jt + 3) * T::kRowBytes;
            s.sov = slot0(jt + 2) * 2;
            s.m0k = lds0 + sk * kW2Slot + wave * T::kInstr * 1024;
            s.m0v = lds0 + kW2VRing + sk2 * kW2Slot + wave * T::vInstr * 1024;
            s.kslot = lds0 + sk1 * kW2Slot;
            s.vslot = sk * kW2Slot;
            pg[0] = pg[1];
            pg[1] = pg[2];
            pg[2] = pk;
            // The next page id is requested only after everything above has
            // consumed the older ones: scalar loads complete out of order, so
            // a use of an older id waits for every load in flight.
            asm volatile("" ::"s"(s.rk), "s"(s.rv), "s"(pg[1]), "s"(pg[2]) : "memory");
            pg[3] = jt + 4 < tile_end ? page_at(jt + 4) : -1;
            sk = sk1;
            return s;
        };
        // Bodies jt whose next tile every row of the unit sees whole (no mask,
        // no V^T fix-up) and whose DMA stays inside the unit's run go through
        // w2_run: jt in [run_lo, run_hi).
        auto floor_div = [](int64_t a, int64_t b) { return a >= 0 ? a / b : -((-a + b - 1) / b); };
        int64_t full_lo = -floor_div(-static_cast<int64_t>(zero_lo), kBK);   // first key at or above zero_lo
        if (window) full_lo = max(full_lo, -floor_div(-(static_cast<int64_t>(last_pos) - window + 1 - k_pos0), kBK));
        const int64_t full_hi = min(floor_div(static_cast<int64_t>(first_pos) - (kBK - 1) - k_pos0, kBK) + 1,
                                    floor_div(zero_hi, kBK));
        const int run_lo = static_cast<int>(max<int64_t>(full_lo - 1, tile_beg));
        const int run_hi = static_cast<int>(min<int64_t>(full_hi - 1, tile_end - 3));
        W2Run rn;
        {
            // every field wave-uniform and in SGPRs (the asm takes them as such)
            auto u = [](auto x) { return static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<int>(x))); };
            const uint64_t kp = reinterpret_cast<uint64_t>(kpool), vp = reinterpret_cast<uint64_t>(vpool);
            rn.kbase = u(lds0);
            rn.m0k = u(lds0 + wave * T::kInstr * 1024);
            rn.m0v = u(lds0 + kW2VRing + wave * T::vInstr * 1024);
            rn.pages = pages;
            rn.kplo = u(kp), rn.kphi = u(kp >> 32);
            rn.vdlo = u(vp - kp), rn.vdhi = u((vp - kp) >> 32);
            rn.pbytes = u(static_cast<unsigned>(T::kRowBytes) << log2P);
            rn.npg = num_pages;
            rn.lastlp = u(n_pages - 1);
            rn.log2p = u(log2P);
            rn.pmask = u((1u << log2P) - 1);
        }
        for (int jt = tile_beg;;) {
            const bool odd = ((jt - tile_beg) & 1) != 0;
            if (jt + 1 >= tile_end) {
                W2Step s;
                s.kslot = lds0;
                s.vslot = sk * kW2Slot;
                if (odd)
                    w2_last_y(m0, m1, l0, l1, ad, s, scale_log2);
                else
                    w2_last_x(m0, m1, l0, l1, ad, s, scale_log2);
                break;
            }
            if (jt >= run_lo && jt + 2 <= run_hi) {
                unsigned cnt = static_cast<unsigned>(run_hi - jt), kk = static_cast<unsigned>((jt + 3) * kBK);
                int idk = pg[3], idv = pg[2];
                w2_run(m0, m1, l0, l1, ad, rn, static_cast<unsigned>((jt - tile_beg) % 6), cnt, kk, idk, idv,
                       scale_log2);
                jt = run_hi;
                pg[2] = jt + 2 < tile_end ? idv : -1;
                pg[3] = jt + 3 < tile_end ? idk : -1;
                sk = static_cast<unsigned>((jt - tile_beg) % 3);
                continue;
            }
            const unsigned vs1 = sk == 2 ? 0 : sk + 1;   // V slot of tile jt+1
            const W2Step s = step(jt);
            if (odd)
                w2_tile_yx(m0, m1, l0, l1, ad, s, mask(jt + 1), scale_log2);
            else
                w2_tile_xy(m0, m1, l0, l1, ad, s, mask(jt + 1), scale_log2);
            if (edge_tile(jt + 1)) {
                fixup(vs1, jt + 1);
                __syncthreads();
            }
            ++jt;
        }
    }

    if (tile_beg >= tile_end) {   // no tile (no unit the builder makes): O and the partial result are zero
        request();
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        publish();
        __syncthreads();
        nxt = __builtin_amdgcn_readfirstlane(next_word[0]);
    }

    // Epilogue: lane (col, half) holds O^T dims 32 db + 8 j + 4 half + i of its
    // column of block k as the four values w2_get_o<k, db, j> returns. Stored
    // from there, one store instruction would put 16 or 32 bytes into each of
    // 32 rows, 32 cache lines per instruction. So each wave stages a block
    // row-major in LDS and stores whole rows, 1 KB contiguous per instruction
    // in a row of O, or in a run of partial-result rows.
    w2_drain();
    const float ltot[2] = {sum_halves(l0), sum_halves(l1)};
    const float mfin[2] = {m0, m1};
    // The rings become the staging area once every wave is past its last
    // tile and the transfers of the tiles past the run (zeros) have landed.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    char *const stage = smem + wave * (kWaveRows * D * 4);   // this wave's 16 KB
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    // Block k through the staging area, one dim block at a time straight from
    // its accumulators: row r at r * RB, its 16-byte chunk c at chunk position
    // c ^ (r & 15), which spreads the 32 rows one write instruction touches
    // over the LDS banks. Values are multiplied by sc (in fp32) and rounded
    // to the element type; row r goes to dst0 + r * stride, rows at or past
    // nrows do not exist.
    auto put_rows = [&](auto k_c, auto f32_c, float sc, char *dst0, int64_t stride, int nrows) {
        constexpr int k = decltype(k_c)::value;
        constexpr bool F32 = decltype(f32_c)::value;
        constexpr int EB = F32 ? 4 : 2, RB = D * EB, CH = RB / 16, RPP = 1024 / RB, NP = kWaveRows / RPP;
        asm volatile("" ::: "memory");   // after the previous block's reads
        auto put_db = [&](auto db_c) {
            constexpr int db = decltype(db_c)::value;
            float4 v[4];
            w2_get_o<k, db, 0>(v[0].x, v[0].y, v[0].z, v[0].w);
            w2_get_o<k, db, 1>(v[1].x, v[1].y, v[1].z, v[1].w);
            w2_get_o<k, db, 2>(v[2].x, v[2].y, v[2].z, v[2].w);
            w2_get_o<k, db, 3>(v[3].x, v[3].y, v[3].z, v[3].w);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int b0 = (32 * db + 8 * jj + 4 * half) * EB;   // byte offset within the row
                char *p = stage + col * RB + (((b0 >> 4) ^ (col & 15)) << 4) + (b0 & 15);
                const float4 x = v[jj];
                if constexpr (F32)
                    *reinterpret_cast<f32x4 *>(p) = f32x4{x.x * sc, x.y * sc, x.z * sc, x.w * sc};
                else
                    *reinterpret_cast<bf16x4 *>(p) =
                        bf16x4{static_cast<__bf16>(x.x * sc), static_cast<__bf16>(x.y * sc),
                               static_cast<__bf16>(x.z * sc), static_cast<__bf16>(x.w * sc)};
            }
        };
        put_db(std::integral_constant<int, 0>{});
        put_db(std::integral_constant<int, 1>{});
        put_db(std::integral_constant<int, 2>{});
        put_db(std::integral_constant<int, 3>{});
        // Lanes read rows other lanes wrote: one wavefront's LDS operations
        // complete in order, so only the compiler has to keep them so. Lane
        // (rl, c) moves chunk c of rows rl, rl + RPP, ..., four reads in
        // flight before their stores.
        asm volatile("" ::: "memory");
        const int rl = lane / CH, c = lane % CH;
        char *g = dst0 + rl * stride + 16 * c;
#pragma unroll
        for (int p0 = 0; p0 < NP; p0 += 4) {
            u32x4 x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = (p0 + i) * RPP + rl;
                x[i] = *reinterpret_cast<const u32x4 *>(stage + r * RB + ((c ^ (r & 15)) << 4));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if ((p0 + i) * RPP + rl < nrows) *reinterpret_cast<u32x4 *>(g + (p0 + i) * RPP * stride) = x[i];
        }
    };
    auto finish = [&](auto k_c) {
        constexpr int k = decltype(k_c)::value;
        if (part >= 0) {
            constexpr int kPairs = kUnitRows * HPW;
            float *slot = parts + static_cast<int64_t>(part) * (kPairs * (D + 2));
            const int rr0 = hoff[k] * kUnitRows + rblk[k] * kWaveRows;   // the block's first slot row
            put_rows(k_c, std::true_type{}, 1.0f, reinterpret_cast<char *>(slot + static_cast<int64_t>(rr0) * D),
                     D * 4, kWaveRows);
            if (half == 0) {
                slot[kPairs * D + rr0 + col] = mfin[k];
                slot[kPairs * (D + 1) + rr0 + col] = ltot[k];
            }
            return;
        }
        const float inv = ltot[k] > 0.f ? 1.0f / ltot[k] : 0.f;
        constexpr int EB = OUT_BF16 ? 2 : 4;
        const int64_t grow0 = static_cast<int64_t>(q_row0) + wrow0[k];   // the block's first row of O
        const int nrows = blk_ok[k] ? static_cast<int>(min<int64_t>(n_q - wrow0[k], total_q_rows - grow0)) : 0;
        put_rows(k_c, std::integral_constant<bool, !OUT_BF16>{}, inv,
                 static_cast<char *>(o) + (grow0 * hq + head[k]) * D * EB, static_cast<int64_t>(hq) * D * EB, nrows);
        if (lse && half == 0 && row_ok[k])
            lse[static_cast<int64_t>(head[k]) * total_q_rows + my_row[k]] =
                (mfin[k] + __log2f(ltot[k])) * 0.69314718055994530942f;
    };
    finish(std::integral_constant<int, 0>{});
    finish(std::integral_constant<int, 1>{});
    }   // valid unit
    }
    if (nxt >= num_units) break;
    u = nxt;
    }
}

// Decode / small-chunk kernel (pages of at least one tile). A unit is one
// segment's few new rows for all G query heads of its KV head: column c of
// the MFMAs is the (row c / G, head c % G) pair, so the 32 columns carry up to
// 32 / G rows. The step is bound by HBM bandwidth. Each workgroup is a single
// wavefront that streams its unit's 64-key tiles straight from the pages into
// its MFMA operand registers, loading the next tile while it computes the
// current one; eight such workgroups share a CU, so one wave's start (reading
// its unit's descriptors, Q and page ids) and finish (writing its result)
// overlap the other waves' streaming, and no wave waits for another.
constexpr int kDecThreads = 64;

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kDecThreads, 2) void attn_decode_kernel(
    const u16 *__restrict__ q, const u16 *__restrict__ kpool, const u16 *__restrict__ vpool, int64_t num_pages,
    int log2P, const int32_t *__restrict__ seg_desc, const int32_t *__restrict__ page_list,
    int64_t num_page_entries, const int32_t *__restrict__ work, int32_t num_segments, int32_t total_q_rows,
    int32_t hq, int32_t unit_rows, int32_t unit_heads, float scale_log2, void *__restrict__ o,
    float *__restrict__ lse, float *__restrict__ parts, int32_t num_parts)
{
    constexpr int kSteps = D / 16;
    constexpr int kDBlocks = D / 32;
    constexpr int kQLd = D + 8;    // bf16 per Q^T column row: 16-byte pad, so the lanes' reads hit distinct banks
    constexpr int kIdCap = 1024;   // page ids staged per pass
    __shared__ __attribute__((aligned(16))) u16 qlds[kWaveRows * kQLd];
    __shared__ int32_t ids[kIdCap];

    const int32_t *urec = work + static_cast<int64_t>(blockIdx.x) * SEGKV_UNIT_FIELDS;
    const i32x4 unit = *reinterpret_cast<const i32x4 *>(urec);
    const i32x4 unit2 = *reinterpret_cast<const i32x4 *>(urec + 4);
    const int seg = unit[SEGKV_UNIT_SEGMENT], row0 = unit[SEGKV_UNIT_ROW0], head0 = unit[SEGKV_UNIT_HEAD0];
    const int run0 = unit2[SEGKV_UNIT_TILE0 - 4], run_len = unit[SEGKV_UNIT_TILES];
    const int part = unit2[SEGKV_UNIT_PART - 4];
    if (seg < 0 || seg >= num_segments || part >= num_parts || unit_heads < 1 || unit_rows < 1 ||
        unit_rows * unit_heads > kWaveRows)
        return;
    const int32_t *desc = seg_desc + static_cast<int64_t>(seg) * SEGKV_SEG_FIELDS;
    const int q_row0 = desc[SEGKV_SEG_Q_ROW0], n_q = desc[SEGKV_SEG_N_Q], q_pos0 = desc[SEGKV_SEG_Q_POS0];
    const int window = desc[SEGKV_SEG_WINDOW], k_pos0 = desc[SEGKV_SEG_K_POS0], k_len = desc[SEGKV_SEG_K_LEN];
    const int page_off = desc[SEGKV_SEG_PAGE_OFF];
    // k_pos0 starts a page, so a 64-key tile never crosses one.
    if (row0 < 0 || row0 >= n_q || page_off < 0 || page_off >= num_page_entries || k_len < 1 ||
        (k_pos0 & ((1 << log2P) - 1)) != 0)
        return;
    int n_pages = (k_len + (1 << log2P) - 1) >> log2P;
    if (n_pages > num_page_entries - page_off) n_pages = static_cast<int>(num_page_entries - page_off);
    const int32_t *pages = page_list + page_off;
    const int P = 1 << log2P;

    const int lane = threadIdx.x;
    const int col = lane & 31, half = lane >> 5;

    // Rows of the unit and its band of tiles, cut to the unit's run.
    const int unit_end = min(row0 + unit_rows, n_q);
    const int first_pos = q_pos0 + row0, last_pos = q_pos0 + unit_end - 1;
    const int lo_pos = window ? max(0, first_pos - window + 1) : 0;
    const int tile_beg = max((lo_pos - k_pos0) / kBK, run0);
    const int tile_end = min((last_pos + 1 - k_pos0 + kBK - 1) / kBK, run0 + max(run_len, 0));
    const int zero_lo = max(0, (window ? max(0, q_pos0 - window + 1) : 0) - k_pos0);   // stored and visible keys
    const int zero_hi = k_len;

    // This lane's column: (row, head) pair, its query position and the keys it
    // may see inside the run.
    const int my_t = min(row0 + col / unit_heads, n_q - 1);
    const int my_pos = q_pos0 + my_t;
    const int run_lo = k_pos0 + tile_beg * kBK, run_hi = k_pos0 + tile_end * kBK - 1;
    const int lo_eff = max(window ? my_pos - window + 1 : 0, run_lo);
    const int hi_eff = min(my_pos, run_hi);
    const int all_lo = max(window ? last_pos - window + 1 : 0, run_lo);
    const int all_hi = min(first_pos, run_hi);

    const u16 *qcol = qlds + col * kQLd + 8 * half;
    f32x16 oacc[kDBlocks];
#pragma unroll
    for (int i = 0; i < kDBlocks; ++i) oacc[i] = f32x16{};
    float m = kNegBig, lsum = 0.f;

    // Page ids of the run, staged in LDS a pass of kIdCap pages at a time
    // (k_pos0 starts a page, so entry e holds keys e P .. e P + P - 1).
    const int tiles_per_page = P / kBK;
    const int tiles_per_pass = kIdCap * tiles_per_page;

    // One 64-key tile's operands, read from its page with buffer loads (a
    // missing page or a tile past the pass has an empty range: zeros, no
    // traffic; every path issues the same loads, so the compiler's waits
    // before a use count only that tile's loads). Each batch of V loads covers
    // whole 128-byte lines of the V^T rows: reading the two halves of a line
    // far apart in time costs HBM efficiency. K: the A operand of
    // S^T = K . Q^T for keys 32 g + swizzle_row(col) (so S^T registers are the
    // P^T operand), 8 dims at 16 s + 8 half. V^T: the A operand of
    // O^T += V^T . P^T, row d = 32 db + col, keys 16 t + 8 half .. + 7.
    bf16x8 kreg[2][kSteps];
    bf16x8 vreg[4][kDBlocks];
    const unsigned k_lane = static_cast<unsigned>((swizzle_row(col) * D + 8 * half) * 2);
    const unsigned v_lane = static_cast<unsigned>((col * P + 8 * half) * 2);
    int pass_end = 0, id0 = 0;
    auto page_of = [&](int tile) -> int {
        int page = -1;
        if (tile < pass_end) page = __builtin_amdgcn_readfirstlane(ids[tile / tiles_per_page - id0]);
        return page;
    };
    auto fetch_k_pg = [&](int page, int tile) {
        const int pg = max(page, 0);
        const __amdgpu_buffer_rsrc_t rk =
            page_rsrc(kpool + ((static_cast<int64_t>(pg) * D) << log2P), page >= 0 ? ((D * 2) << log2P) : 0);
        const unsigned off = k_lane + static_cast<unsigned>(((tile * kBK) & (P - 1)) * D * 2);
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int s = 0; s < kSteps; ++s)
                kreg[g][s] = __builtin_bit_cast(
                    bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, off + 32 * g * D * 2 + 32 * s, 0, 0));
    };
    auto fetch_v_pg = [&](int page, int tile) {
        const int pg = max(page, 0);
        const __amdgpu_buffer_rsrc_t rv =
            page_rsrc(vpool + ((static_cast<int64_t>(pg) * D) << log2P), page >= 0 ? ((D * 2) << log2P) : 0);
        const unsigned off = v_lane + static_cast<unsigned>(((tile * kBK) & (P - 1)) * 2);
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                vreg[t][db] = __builtin_bit_cast(
                    bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, off + 64 * db * P + 32 * t, 0, 0));
    };

    auto fetch_k = [&](int tile) { fetch_k_pg(page_of(tile), tile); };
    auto fetch_v = [&](int tile) { fetch_v_pg(page_of(tile), tile); };

    // One tile: S^T, then the next tile's K is requested; the softmax; P V,
    // then the next tile's V is requested.
    auto compute = [&](int tile) {
        const int key0 = tile * kBK;
        f32x16 sacc[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            sacc[g] = f32x16{};
#pragma unroll
            for (int s = 0; s < kSteps; ++s)
                sacc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    kreg[g][s], *reinterpret_cast<const bf16x8 *>(qcol + 16 * s), sacc[g], 0, 0, 0);
        }
        fetch_k(tile + 1);
        const int kp0 = k_pos0 + key0;
        const bool live = tile < pass_end;   // a tile past the pass belongs to the next one
        if (!(live && kp0 >= all_lo && kp0 + kBK - 1 <= all_hi)) {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const int kbase = kp0 + 32 * g + 8 * half;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int pos = kbase + 16 * (e >> 3) + (e & 7);
                    sacc[g][e] = (live && pos >= lo_eff && pos <= hi_eff) ? sacc[g][e] : -__builtin_inff();
                }
            }
        }
        float mx = vmax(sacc[0][0], sacc[0][1]);
#pragma unroll
        for (int e = 2; e < 16; e += 2) mx = vmax(vmax(mx, sacc[0][e]), sacc[0][e + 1]);
#pragma unroll
        for (int e = 0; e < 16; e += 2) mx = vmax(vmax(mx, sacc[1][e]), sacc[1][e + 1]);
        const float mt = max_halves(mx) * scale_log2;
        if (__any(mt > m + kRescaleSlack)) {
            const float m_new = fmaxf(m, mt);
            const float alpha = __builtin_amdgcn_exp2f(m - m_new);
            lsum *= alpha;
#pragma unroll
            for (int i = 0; i < kDBlocks; ++i) oacc[i] *= alpha;
            m = m_new;
        }
        // V entries outside the stored-and-visible range may hold anything
        // (0 * NaN would reach O): clear them on the tiles that have any.
        if (key0 < zero_lo || key0 + kBK > zero_hi) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                u32x4 keep;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int idx = key0 + 16 * t + 8 * half + 2 * w;
                    keep[w] = ((idx >= zero_lo && idx < zero_hi) ? 0xffffu : 0u) |
                              ((idx + 1 >= zero_lo && idx + 1 < zero_hi) ? 0xffff0000u : 0u);
                }
#pragma unroll
                for (int db = 0; db < kDBlocks; ++db)
                    vreg[t][db] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, vreg[t][db]) & keep);
            }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bf16x8 pb;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                pb[i] = static_cast<__bf16>(
                    __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t >> 1][8 * (t & 1) + i], scale_log2, -m)));
            lsum = sum8_bf16(pb, lsum);
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vreg[t][db], pb, oacc[db], 0, 0, 0);
        }
        fetch_v(tile + 1);
    };

    // Passes over the pages of each kIdCap-page stretch of the segment, one
    // tile per step (the tile past a pass is requested as an empty range).
    // The first pass takes its first tile's page by a scalar load, so that
    // tile's K and V requests go out right after Q's and beside the ids'
    // instead of after them.
    // Q^T, the B operand (lane column = pair), sits in LDS for the loop. All
    // of a lane's chunks are requested before any is written (one round trip,
    // not one per chunk).
    // Buffer loads over the unit's rows of Q: a lane with nothing to load
    // gets an offset past the range and reads zeros, so no load sits behind a
    // branch (which would make the compiler wait for each before the next).
    constexpr int kQChunks = kWaveRows * (D / 8) / kDecThreads;
    const int64_t qrow0 = static_cast<int64_t>(q_row0) + row0;
    const int q_rows = static_cast<int>(max<int64_t>(0, min<int64_t>(unit_end - row0, total_q_rows - qrow0)));
    const __amdgpu_buffer_rsrc_t rq = page_rsrc(q + qrow0 * hq * D, q_rows * hq * D * 2);
    u32x4 qraw[kQChunks];
#pragma unroll
    for (int c = 0; c < kQChunks; ++c) {
        const int i = lane + c * kDecThreads;
        const int qc = i / (D / 8), qd = 8 * (i % (D / 8));
        const int qr = qc / unit_heads, qh = qc % unit_heads;
        const bool ok = qc < unit_rows * unit_heads && qr < q_rows && head0 + qh < hq;
        const unsigned off = ok ? static_cast<unsigned>(((qr * hq + head0 + qh) * D + qd) * 2) : 0x80000000u;
        qraw[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
    }
#pragma unroll
    for (int c = 0; c < kQChunks; ++c) {
        const int i = lane + c * kDecThreads;
        *reinterpret_cast<u32x4 *>(qlds + (i / (D / 8)) * kQLd + 8 * (i % (D / 8))) = qraw[c];
    }
    int pass_beg = tile_beg;
    pass_end = min(tile_end, (pass_beg / tiles_per_pass + 1) * tiles_per_pass);
    id0 = pass_beg / tiles_per_page;
    {
        int pg0 = -1;
        if (tile_beg < tile_end && id0 < n_pages) {
            const int v = pages[id0];
            pg0 = (v >= 0 && v < num_pages) ? v : -1;
        }
        fetch_k_pg(pg0, pass_beg);
        fetch_v_pg(pg0, pass_beg);
    }
    auto stage_ids = [&]() {
        const int n_ids = (pass_end - 1) / tiles_per_page - id0 + 1;
        for (int i = lane; i < n_ids; i += kDecThreads) {
            int page = -1;
            if (id0 + i < n_pages) page = pages[id0 + i];
            ids[i] = (page >= 0 && page < num_pages) ? page : -1;
        }
    };
    stage_ids();
    __syncthreads();   // Q^T and the ids are visible to every lane
    for (int tile = pass_beg; tile < pass_end; ++tile) compute(tile);
    __syncthreads();   // every lane is done with the ids before a next pass rewrites them
    for (pass_beg = pass_end; pass_beg < tile_end; pass_beg = pass_end) {
        pass_end = min(tile_end, (pass_beg / tiles_per_pass + 1) * tiles_per_pass);
        id0 = pass_beg / tiles_per_page;
        stage_ids();
        __syncthreads();
        fetch_k(pass_beg);
        fetch_v(pass_beg);
        for (int tile = pass_beg; tile < pass_end; ++tile) compute(tile);
        __syncthreads();
    }

    // Results straight from the O^T registers: lane (col, half) holds dims
    // 32 db + 8 j + 4 half + i of pair col as oacc[db][4 j + i].
    const float ltot = sum_halves(lsum);
    const int cr = col / unit_heads, ch = col % unit_heads;
    if (col >= unit_rows * unit_heads || row0 + cr >= n_q || head0 + ch >= hq) return;
    const int64_t row = static_cast<int64_t>(q_row0) + row0 + cr;
    if (row >= total_q_rows) return;
    const int hd = head0 + ch;
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    if (part >= 0) {
        const int pairs = unit_rows * unit_heads, r = ch * unit_rows + cr;
        float *slot = parts + static_cast<int64_t>(part) * pairs * (D + 2);
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<f32x4 *>(slot + r * D + 32 * db + 8 * j + 4 * half) =
                    f32x4{oacc[db][4 * j], oacc[db][4 * j + 1], oacc[db][4 * j + 2], oacc[db][4 * j + 3]};
        if (half == 0) {
            slot[pairs * D + r] = m;
            slot[pairs * (D + 1) + r] = ltot;
        }
        return;
    }
    const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
    const int64_t obase = (row * hq + hd) * D + 4 * half;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4 v = f32x4{oacc[db][4 * j], oacc[db][4 * j + 1], oacc[db][4 * j + 2], oacc[db][4 * j + 3]} * inv;
            const int64_t at = obase + 32 * db + 8 * j;
            if constexpr (OUT_BF16) {
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                *reinterpret_cast<bf16x4 *>(static_cast<u16 *>(o) + at) =
                    bf16x4{static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1]), static_cast<__bf16>(v[2]),
                           static_cast<__bf16>(v[3])};
            } else {
                *reinterpret_cast<f32x4 *>(static_cast<float *>(o) + at) = v;
            }
        }
    if (lse && half == 0)
        lse[static_cast<int64_t>(hd) * total_q_rows + row] = (m + __log2f(ltot)) * 0.69314718055994530942f;
}

// Attention mass of the step's new tokens (RedKnot summary page, "Sparse
// FFN": the tokens with the highest attention scores get the dense FFN). A
// second pass over the same units, after the attention has produced the LSE:
// S = Q . K^T with Q as the A operand, so each lane owns one key column and
// its accumulator registers are query rows; p = exp(s - lse) then sums over
// the queries inside the lane, plus one exchange between the two 32-lane
// halves. Each wave adds its 64 column sums to mass[] with float atomics
// (several heads, row blocks and KV heads reach the same token). Only K is
// staged; keys before the step (cached tokens) are not visited.
template <int D, int HPW, int NW>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attn_mass_kernel(
    const u16 *__restrict__ q, const u16 *__restrict__ kpool, int64_t num_pages, int log2P,
    const int32_t *__restrict__ seg_desc, const int32_t *__restrict__ page_list, int64_t num_page_entries,
    const int32_t *__restrict__ work, int32_t num_segments, int32_t total_q_rows, int32_t hq, float scale_log2,
    const float *__restrict__ lse, float *__restrict__ mass)
{
    using T = DmaTile<D, NW>;
    constexpr int kRowBlocks = NW / HPW;
    constexpr int kUnitRows = kWaveRows * kRowBlocks;
    constexpr int kSteps = D / 16;
    __shared__ __attribute__((aligned(1024))) char kst0[T::kBytes];
    __shared__ __attribute__((aligned(1024))) char kst1[T::kBytes];

    const int32_t *urec = work + static_cast<int64_t>(blockIdx.x) * SEGKV_UNIT_FIELDS;
    const i32x4 unit = *reinterpret_cast<const i32x4 *>(urec);
    const i32x4 unit2 = *reinterpret_cast<const i32x4 *>(urec + 4);
    const int seg = unit[SEGKV_UNIT_SEGMENT], row0 = unit[SEGKV_UNIT_ROW0], head0 = unit[SEGKV_UNIT_HEAD0];
    const int run0 = unit2[SEGKV_UNIT_TILE0 - 4], run_len = unit[SEGKV_UNIT_TILES];
    if (seg < 0 || seg >= num_segments) return;
    const int32_t *desc = seg_desc + static_cast<int64_t>(seg) * SEGKV_SEG_FIELDS;
    const int q_row0 = desc[SEGKV_SEG_Q_ROW0], n_q = desc[SEGKV_SEG_N_Q], q_pos0 = desc[SEGKV_SEG_Q_POS0];
    const int window = desc[SEGKV_SEG_WINDOW], k_pos0 = desc[SEGKV_SEG_K_POS0], k_len = desc[SEGKV_SEG_K_LEN];
    const int page_off = desc[SEGKV_SEG_PAGE_OFF];
    if (row0 < 0 || row0 >= n_q || page_off < 0 || page_off >= num_page_entries || k_len < 1 || q_pos0 < k_pos0)
        return;
    int n_pages = (k_len + (1 << log2P) - 1) >> log2P;
    if (n_pages > num_page_entries - page_off) n_pages = static_cast<int>(num_page_entries - page_off);
    const int32_t *pages = page_list + page_off;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const int head = head0 + wave % HPW;
    const int wrow0 = row0 + (wave / HPW) * kWaveRows;

    const int unit_end = min(row0 + kUnitRows, n_q);
    const int first_pos = q_pos0 + row0, last_pos = q_pos0 + unit_end - 1;
    const int lo_pos = window ? max(0, first_pos - window + 1) : 0;
    // the unit's run, from the first tile holding a new token
    const int tile_beg = max(max((lo_pos - k_pos0) / kBK, run0), (q_pos0 - k_pos0) / kBK);
    const int tile_end = min((last_pos + 1 - k_pos0 + kBK - 1) / kBK, run0 + max(run_len, 0));
    const int key_end = k_pos0 + k_len;   // one past the last stored key (the step's last token)

    const bool wave_valid = wrow0 < n_q && head < hq;
    const int wrow_end = min(wrow0 + kWaveRows, n_q);
    const int wp_lo = q_pos0 + wrow0, wp_hi = q_pos0 + max(wrow_end, wrow0 + 1) - 1;

    // A operand: query row `col`, 8 dims per k-step (the same registers as the
    // B operand of the attention kernel).
    bf16x8 qreg[kSteps];
    {
        const int my_t = min(wrow0 + col, n_q - 1);
        const int64_t my_row = static_cast<int64_t>(q_row0) + my_t;
        const bool can_load = wave_valid && my_row < total_q_rows;
        const u16 *qp = q + (my_row * hq + min(head, hq - 1)) * D + 8 * half;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (can_load) raw = *reinterpret_cast<const u32x4 *>(qp + 16 * s);
            qreg[s] = __builtin_bit_cast(bf16x8, raw);
        }
    }
    // The query rows of this lane's accumulator registers: e -> 8 (e / 4) +
    // 4 half + e % 4. Their LSE in log2 units (+inf: row absent, weight 0).
    float lse2[16];
    int qpos[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int t = wrow0 + 8 * (e >> 2) + 4 * half + (e & 3);
        const bool ok = wave_valid && t < n_q && static_cast<int64_t>(q_row0) + t < total_q_rows;
        lse2[e] = ok ? lse[static_cast<int64_t>(head) * total_q_rows + q_row0 + t] * 1.44269504088896340736f
                     : __builtin_inff();
        qpos[e] = q_pos0 + t;
    }

    int win = ((tile_beg * kBK) >> log2P) >> 6;
    auto load_window = [&](int w) { return pages[min(w * 64 + lane, n_pages - 1)]; };
    int win_cur = load_window(win), win_next = load_window(win + 1);
    auto tile_page = [&](int jt) {
        const int lp = (jt * kBK) >> log2P;
        if ((lp >> 6) != win) {
            win = lp >> 6;
            win_cur = win_next;
            win_next = load_window(win + 1);
        }
        const int id = __builtin_amdgcn_readlane(win_cur, lp & 63);
        return (lp < n_pages && id >= 0 && id < num_pages) ? id : -1;
    };
    unsigned kdma[T::kInstr];
#pragma unroll
    for (int i = 0; i < T::kInstr; ++i) {
        const int p = (wave * T::kInstr + i) * 1024 + lane * 16;
        const int r = p / T::kRowBytes, c = ((p % T::kRowBytes) / 16) ^ kswz<D>(r);
        kdma[i] = static_cast<unsigned>(r * T::kRowBytes + c * 16);
    }
    auto dma_k = [&](char *dst, int jt) {
        const int page = tile_page(jt);
        const unsigned slot0 = static_cast<unsigned>((jt * kBK) & ((1 << log2P) - 1));
        const int64_t pg = page >= 0 ? page : 0;
        const __amdgpu_buffer_rsrc_t rk =
            page_rsrc(kpool + ((pg * D) << log2P), page >= 0 ? (T::kRowBytes << log2P) : 0);
#pragma unroll
        for (int i = 0; i < T::kInstr; ++i)
            dma16(rk, dst + (wave * T::kInstr + i) * 1024, kdma[i], slot0 * T::kRowBytes);
    };

    auto compute = [&](const char *kt, int jt) {
        const int kp0 = k_pos0 + jt * kBK;
        const bool full = kp0 >= q_pos0 && kp0 + kBK <= key_end && kp0 + kBK - 1 <= wp_lo &&
                          (window == 0 || kp0 >= wp_hi - window + 1);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = 32 * h + col;   // key row of this lane's column
            f32x16 sacc = {};
#pragma unroll
            for (int s = 0; s < kSteps; ++s) {
                const bf16x8 b =
                    *reinterpret_cast<const bf16x8 *>(kt + r * T::kRowBytes + (((2 * s + half) ^ kswz<D>(r)) << 4));
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qreg[s], b, sacc, 0, 0, 0);
            }
            const int kpos = kp0 + r;
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e], scale_log2, -lse2[e]));
                if (!full) {
                    const bool vis = kpos <= qpos[e] && (window == 0 || qpos[e] - kpos < window) &&
                                     kpos >= q_pos0 && kpos < key_end;
                    p = vis ? p : 0.f;
                }
                acc += p;
            }
            float lo, hi;
            swap_halves(acc, lo, hi);
            const float tot = lo + hi;
            if (half == 0 && wave_valid && kpos >= q_pos0 && kpos < key_end)
                atomicAdd(mass + q_row0 + (kpos - q_pos0), tot);
        }
    };

    if (tile_beg < tile_end) {
        dma_k(kst0, tile_beg);
        __syncthreads();
        int jt = tile_beg;
        auto iteration = [&](int j, char *cur, char *nxt) {
            if (j + 1 < tile_end) dma_k(nxt, j + 1);
            compute(cur, j);
            __syncthreads();
        };
        for (; jt + 1 < tile_end; jt += 2) {
            iteration(jt, kst0, kst1);
            iteration(jt + 1, kst1, kst0);
        }
        if (jt < tile_end) iteration(jt, kst0, kst1);
    }
}

__global__ void fill_zero_kernel(float *__restrict__ x, int64_t n)
{
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        x[i] = 0.f;
}

// Merge pass for split blocks (split-KV): kMergeDSplit workgroups per merge
// entry, each for a quarter of the head dim. The runs' partial results
// combine exactly as blocks of one online softmax:
// O = sum_r 2^(m_r - M) O_r / sum_r 2^(m_r - M) l_r with M the largest m_r.
// Every lane owns four consecutive dims of one valid (row, head) pair and
// folds a stride of the runs into a running (M, L, O) in one pass (several
// lanes per item when the block has few pairs, combined in LDS the same way),
// so a wave reads whole rows of the partials, the loads of many runs overlap,
// and the entry itself carries the output rows (no segment lookup).
constexpr int kMergeDSplit = 4;

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void merge_parts_kernel(
    const int32_t *__restrict__ merge, const float *__restrict__ parts, int32_t num_parts, int32_t unit_rows,
    int32_t unit_heads, int32_t total_q_rows, int32_t hq, void *__restrict__ o, float *__restrict__ lse)
{
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    __shared__ float red_m[kThreads], red_l[kThreads];
    __shared__ f32x4 red_o[kThreads];
    const int32_t *e = merge + static_cast<int64_t>(blockIdx.x) * SEGKV_MERGE_FIELDS;
    const int head0 = e[SEGKV_MERGE_HEAD0], part0 = e[SEGKV_MERGE_PART0], nparts = e[SEGKV_MERGE_NPARTS];
    const int out_row0 = e[SEGKV_MERGE_OUT_ROW0], rows_ok = e[SEGKV_MERGE_ROWS];
    const int pairs = unit_rows * unit_heads;
    const int heads_ok = min(unit_heads, hq - head0);
    if (part0 < 0 || nparts < 1 || part0 > num_parts - nparts || rows_ok < 1 || rows_ok > unit_rows ||
        out_row0 < 0 || out_row0 > total_q_rows - rows_ok || head0 < 0 || heads_ok < 1 || pairs > kThreads)
        return;
    const int nv = rows_ok * heads_ok;   // valid pairs, vr = head-major over rows_ok
    const int64_t kSlot = static_cast<int64_t>(pairs) * (D + 2);   // floats per partial result
    const float *base = parts + static_cast<int64_t>(part0) * kSlot;

    // This workgroup's dims: chunks [c0, c0 + kChunks) of four.
    constexpr int kChunks = D / 4 / kMergeDSplit;
    const int c0 = static_cast<int>(blockIdx.y) * kChunks;
    const int items = nv * kChunks, i = threadIdx.x;
    const int groups = items < kThreads ? kThreads / items : 1;   // lanes per item, each over a stride of runs
    const int grp = i / (items < kThreads ? items : kThreads);
    for (int item0 = 0; item0 < items; item0 += kThreads) {
        const int item = item0 + (groups > 1 ? i % items : i);
        const bool mine = item < items && grp < groups;
        const int vr = mine ? item / kChunks : 0, ch = c0 + (mine ? item % kChunks : 0);
        const int r = (vr / rows_ok) * unit_rows + vr % rows_ok;   // the pair's slot in a partial result
        float M = kNegBig, L = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (mine) {
#pragma unroll 4
            for (int p = grp; p < nparts; p += groups) {
                const float *slot = base + p * kSlot;
                const float mp = slot[pairs * D + r], lp = slot[pairs * (D + 1) + r];
                const f32x4 op = *reinterpret_cast<const f32x4 *>(slot + static_cast<int64_t>(r) * D + 4 * ch);
                const float mn = fmaxf(M, mp);
                const float a = __builtin_amdgcn_exp2f(M - mn), w = __builtin_amdgcn_exp2f(mp - mn);
                acc = acc * a + op * w;
                L = L * a + lp * w;
                M = mn;
            }
        }
        if (groups > 1) {
            red_m[i] = M;
            red_l[i] = L;
            red_o[i] = acc;
            __syncthreads();
            if (grp == 0) {
                for (int g = 1; g < groups; ++g) M = fmaxf(M, red_m[g * items + i]);
                L = 0.f;
                acc = f32x4{0.f, 0.f, 0.f, 0.f};
                for (int g = 0; g < groups; ++g) {
                    const float w = __builtin_amdgcn_exp2f(red_m[g * items + i] - M);
                    L += red_l[g * items + i] * w;
                    acc += red_o[g * items + i] * w;
                }
            }
        }
        if (!mine || grp != 0) continue;
        const int head = head0 + vr / rows_ok;
        const int64_t row = static_cast<int64_t>(out_row0) + vr % rows_ok;
        const float inv = L > 0.f ? 1.0f / L : 0.f;
        const f32x4 v = acc * inv;
        const int64_t obase = (row * hq + head) * D + 4 * ch;
        if constexpr (OUT_BF16) {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            *reinterpret_cast<bf16x4 *>(static_cast<u16 *>(o) + obase) =
                bf16x4{static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1]), static_cast<__bf16>(v[2]),
                       static_cast<__bf16>(v[3])};
        } else {
            *reinterpret_cast<f32x4 *>(static_cast<float *>(o) + obase) = v;
        }
        if (lse && ch == 0)
            lse[static_cast<int64_t>(head) * total_q_rows + row] = (M + __log2f(L)) * 0.69314718055994530942f;
    }
}

// Zeroes the persistent kernel's per-XCD queue counters ahead of it on the
// same stream (a kernel, not a memset node, so a captured graph replays it).
__global__ void zero_queue_kernel(int32_t *queue)
{
    if (threadIdx.x < kXcds) queue[threadIdx.x] = 0;
}

// Compute units of the current device, read once per device.
int device_cus(int *cus)
{
    constexpr int kMaxDevices = 256;
    static std::mutex mu;
    static int count[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SEGKV_ERR_HIP, "attn_prefill: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SEGKV_ERR_UNSUPPORTED, "attn_prefill: device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (!count[dev]) {
        int c = 0;
        e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess || c <= 0)
            return fail(SEGKV_ERR_HIP, "attn_prefill: compute unit count of device %d: %s", dev,
                        hipGetErrorString(e));
        count[dev] = c;
    }
    *cus = count[dev];
    return SEGKV_OK;
}

int log2_of(int p)
{
    int l = 0;
    while ((1 << l) < p) ++l;
    return l;
}

template <int D, int HPW, bool OUT_BF16>
int launch(const segkv_config &cfg, const segkv_dev_tables &t, const void *q, void *o, float *lse, float scale_log2,
           float *parts, int32_t *queue, hipStream_t stream)
{
    const dim3 grid(static_cast<unsigned>(t.num_units)), block(kThreads);
    const u16 *qh = static_cast<const u16 *>(q), *kp = static_cast<const u16 *>(cfg.k_pool);
    const u16 *vp = static_cast<const u16 *>(cfg.v_pool);
    const int log2P = log2_of(cfg.page_size);
    const bool big_page = cfg.page_size >= kBK;
    if (big_page && t.unit_rows * t.unit_heads <= kWaveRows) {
        hipLaunchKernelGGL((attn_decode_kernel<D, OUT_BF16>), grid, dim3(kDecThreads), 0, stream, qh, kp, vp,
                           cfg.num_pages, log2P, t.seg_desc, t.page_list, t.num_page_entries, t.work,
                           t.num_segments, t.total_q_rows, cfg.num_q_heads, t.unit_rows, t.unit_heads, scale_log2,
                           o, lse, parts, t.num_parts);
    } else if (t.unit_heads != HPW) {
        // decode units take any G heads; every prefill kernel is built per heads-per-unit
        return fail(SEGKV_ERR_INVALID_ARG, "attn_prefill: unsupported unit_heads %d", t.unit_heads);
    } else if (big_page && t.unit_rows * t.unit_heads == kWideWaves * kWaveRows) {
        if constexpr (D == 128) {
            // 160 KB of dynamic LDS: above the default limit, set per launch
            // (the attribute is per device; setting it is allowed under graph
            // capture)
            const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_prefill_w2_kernel<HPW, OUT_BF16>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, kW2Lds);
            if (e != hipSuccess) return fail(SEGKV_ERR_HIP, "attn_prefill: LDS attribute: %s", hipGetErrorString(e));
            // Persistent when there are more units than CUs: one workgroup
            // per CU (a multiple of the XCD count), the rest through the
            // per-XCD queues in the workspace, zeroed first.
            int cus = 0;
            const int rc = device_cus(&cus);
            if (rc != SEGKV_OK) return rc;
            const int slots = cus / kXcds * kXcds;
            unsigned nwg = static_cast<unsigned>(t.num_units);
            int32_t *qp = nullptr;
            if (slots > 0 && t.num_units > slots) {
                if (!queue) return fail(SEGKV_ERR_INVALID_ARG, "attn_prefill: no workspace for the work queues");
                hipLaunchKernelGGL(zero_queue_kernel, dim3(1), dim3(64), 0, stream, queue);
                nwg = static_cast<unsigned>(slots);
                qp = queue;
            }
            hipLaunchKernelGGL((attn_prefill_w2_kernel<HPW, OUT_BF16>), dim3(nwg), dim3(4 * 64), kW2Lds, stream, qh,
                               kp, vp, cfg.num_pages, log2P, t.seg_desc, t.page_list, t.num_page_entries, t.work,
                               t.num_units, qp, t.num_segments, t.total_q_rows, cfg.num_q_heads, scale_log2, o, lse,
                               parts, t.num_parts);
        } else
            hipLaunchKernelGGL((attn_prefill_pipe_kernel<D, HPW, OUT_BF16, kWideWaves>), grid, dim3(kWideWaves * 64),
                               0, stream, qh, kp, vp, cfg.num_pages, log2P, t.seg_desc, t.page_list,
                               t.num_page_entries, t.work, t.num_segments, t.total_q_rows, cfg.num_q_heads,
                               scale_log2, o, lse, parts, t.num_parts);
    } else if constexpr (HPW > kWaves) {
        // eight heads per unit exist only in eight-wave (256-pair) units
        return fail(SEGKV_ERR_INVALID_ARG, "attn_prefill: %d heads per unit need units of %d pairs (tables have %d)",
                    HPW, kWideWaves * kWaveRows, t.unit_rows * t.unit_heads);
    } else if (big_page) {
        hipLaunchKernelGGL((attn_prefill_pipe_kernel<D, HPW, OUT_BF16, kWaves>), grid, block, 0, stream, qh, kp, vp,
                           cfg.num_pages, log2P, t.seg_desc, t.page_list, t.num_page_entries, t.work, t.num_segments,
                           t.total_q_rows, cfg.num_q_heads, scale_log2, o, lse, parts, t.num_parts);
    } else {
        hipLaunchKernelGGL((attn_prefill_kernel<D, HPW, OUT_BF16>), grid, block, 0, stream, qh, kp, vp,
                           cfg.num_pages, log2P, t.seg_desc, t.page_list, t.num_page_entries, t.work, t.num_segments,
                           t.total_q_rows, cfg.num_q_heads, scale_log2, o, lse);
    }
    if (t.num_merges > 0)
        hipLaunchKernelGGL((merge_parts_kernel<D, OUT_BF16>), dim3(static_cast<unsigned>(t.num_merges), kMergeDSplit),
                           block, 0, stream, t.merge, parts, t.num_parts, t.unit_rows, t.unit_heads, t.total_q_rows,
                           cfg.num_q_heads, o, lse);
    return SEGKV_OK;
}

template <int D, int HPW>
int launch_dtype(const segkv_config &cfg, const segkv_dev_tables &t, const void *q, void *o, int32_t o_dtype,
                 float *lse, float scale_log2, float *parts, int32_t *queue, hipStream_t stream)
{
    if (o_dtype == SEGKV_DTYPE_BF16) return launch<D, HPW, true>(cfg, t, q, o, lse, scale_log2, parts, queue, stream);
    return launch<D, HPW, false>(cfg, t, q, o, lse, scale_log2, parts, queue, stream);
}

template <int D>
int launch_heads(const segkv_config &cfg, const segkv_dev_tables &t, const void *q, void *o, int32_t o_dtype,
                 float *lse, float scale_log2, float *parts, int32_t *queue, hipStream_t stream)
{
    switch (t.unit_heads) {
    case 8: return launch_dtype<D, 8>(cfg, t, q, o, o_dtype, lse, scale_log2, parts, queue, stream);
    case 4: return launch_dtype<D, 4>(cfg, t, q, o, o_dtype, lse, scale_log2, parts, queue, stream);
    case 2: return launch_dtype<D, 2>(cfg, t, q, o, o_dtype, lse, scale_log2, parts, queue, stream);
    default: return launch_dtype<D, 1>(cfg, t, q, o, o_dtype, lse, scale_log2, parts, queue, stream);
    }
}

template <int D>
void launch_mass(const segkv_config &cfg, const segkv_dev_tables &t, const void *q, const float *lse,
                 float scale_log2, float *mass, hipStream_t stream)
{
    const dim3 grid(static_cast<unsigned>(t.num_units));
    const u16 *qh = static_cast<const u16 *>(q), *kp = static_cast<const u16 *>(cfg.k_pool);
    const int log2P = log2_of(cfg.page_size);
#define SEGKV_MASS(HPW, NW)                                                                                   \
    hipLaunchKernelGGL((attn_mass_kernel<D, HPW, NW>), grid, dim3(NW * 64), 0, stream, qh, kp, cfg.num_pages,    \
                       log2P, t.seg_desc, t.page_list, t.num_page_entries, t.work, t.num_segments,                \
                       t.total_q_rows, cfg.num_q_heads, scale_log2, lse, mass)
    if (t.unit_rows * t.unit_heads == kWideWaves * kWaveRows) {
        switch (t.unit_heads) {
        case 8: SEGKV_MASS(8, kWideWaves); break;
        case 4: SEGKV_MASS(4, kWideWaves); break;
        case 2: SEGKV_MASS(2, kWideWaves); break;
        default: SEGKV_MASS(1, kWideWaves); break;
        }
    } else {
        switch (t.unit_heads) {
        case 4: SEGKV_MASS(4, kWaves); break;
        case 2: SEGKV_MASS(2, kWaves); break;
        default: SEGKV_MASS(1, kWaves); break;
        }
    }
#undef SEGKV_MASS
}

}  // namespace

int launch_attn_mass(const segkv_config &cfg, const segkv_dev_tables &t, const void *q, const float *lse,
                     float scale_log2, float *mass, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();   // a stale error of an earlier, unrelated call is not this call's
    const int64_t n = t.total_q_rows;
    const unsigned blocks = static_cast<unsigned>(std::min<int64_t>((n + kThreads - 1) / kThreads, 1024));
    if (n > 0) hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(kThreads), 0, s, mass, n);
    if (t.num_units > 0) {
        if (cfg.head_dim == 128)
            launch_mass<128>(cfg, t, q, lse, scale_log2, mass, s);
        else
            launch_mass<64>(cfg, t, q, lse, scale_log2, mass, s);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(SEGKV_ERR_HIP, "attn_mass: %s", hipGetErrorString(err));
    return SEGKV_OK;
}

// Split-KV workspace of segkv_attn_prefill_noalloc: one array per device,
// allocated with the code object. In host code `scratch` only names the
// symbol; kernels get the address noalloc_scratch looks up.
static __device__ __align__(256) unsigned char scratch[SEGKV_NOALLOC_SCRATCH_BYTES];

int noalloc_scratch(void **out)
{
    constexpr int kMaxDevices = 256;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SEGKV_ERR_HIP, "attn_prefill_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SEGKV_ERR_UNSUPPORTED, "attn_prefill_noalloc: device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(SEGKV_ERR_HIP, "attn_prefill_noalloc: scratch address on device %d: %s", dev,
                        hipGetErrorString(e));
        addr[dev] = p;
    }
    *out = addr[dev];
    return SEGKV_OK;
}

int launch_attn_prefill(const segkv_config &cfg, const segkv_dev_tables &t, const void *q, void *o,
                        int32_t o_dtype, float *lse, float scale_log2, void *workspace, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *parts = static_cast<float *>(workspace);
    // the work queues follow the partial results (units of 256 pairs only)
    int32_t *queue = workspace && static_cast<int64_t>(t.unit_rows) * t.unit_heads == kWideWaves * kWaveRows
                         ? reinterpret_cast<int32_t *>(static_cast<char *>(workspace) +
                                                       t.num_parts * SEGKV_PART_BYTES(t.unit_rows, t.unit_heads,
                                                                                      cfg.head_dim))
                         : nullptr;
    (void)hipGetLastError();   // a stale error of an earlier, unrelated call is not this call's
    const int rc = cfg.head_dim == 128 ? launch_heads<128>(cfg, t, q, o, o_dtype, lse, scale_log2, parts, queue, s)
                                       : launch_heads<64>(cfg, t, q, o, o_dtype, lse, scale_log2, parts, queue, s);
    if (rc != SEGKV_OK) return rc;
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(SEGKV_ERR_HIP, "attn_prefill: %s", hipGetErrorString(err));
    return SEGKV_OK;
}

}  // namespace segkv
