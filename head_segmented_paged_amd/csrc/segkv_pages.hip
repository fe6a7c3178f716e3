// Paged KV write (BUILDSTATE), RoPE re-alignment of reused K pages and page
// read-back kernels for gfx950.
//
// Pool layout: K page = bf16 [P][D] (slot-major), V page = bf16 [D][P]
// (dimension-major, the key index innermost). Both are one contiguous block
// per page. The write kernel handles one (sequence, KV head, run of up to 64
// positions inside one page) per workgroup: K rows are copied straight
// through with 16-byte vectors;
// V rows are staged through LDS and written back transposed, each lane
// storing 8 consecutive slots of one dimension.
#include <hip/hip_runtime.h>

#include <cmath>

#include "segkv_internal.h"

namespace segkv {
namespace {

typedef unsigned short u16;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// One workgroup per (sequence, KV head, chunk of CS = min(P, 64) consecutive
// positions inside one page). Positions outside [pos0, pos0 + rows) of the
// sequence are left untouched, so a chunk that shares its page with cached
// tokens keeps them.
__global__ __launch_bounds__(kThreads) void write_pages_kernel(
    const u16 *__restrict__ k_new, const u16 *__restrict__ v_new, int64_t num_rows,
    const int32_t *__restrict__ cu_rows, const int32_t *__restrict__ pos0, const int32_t *__restrict__ page_of,
    int32_t hkv, int32_t max_lp, u16 *__restrict__ k_pool, u16 *__restrict__ v_pool, int64_t num_pages,
    int32_t D, int32_t log2P, int32_t log2CS)
{
    extern __shared__ u16 vtile[];  // [CS][D + 8]
    const int32_t P = 1 << log2P, CS = 1 << log2CS;
    const int32_t b = blockIdx.y / hkv, g = blockIdx.y % hkv;
    const int64_t r_beg = cu_rows[b], r_end = cu_rows[b + 1];
    const int64_t p0 = pos0[b];
    if (r_beg < 0 || r_end <= r_beg || p0 < 0) return;
    const int64_t cx = (p0 >> log2CS) + blockIdx.x;     // chunk index in position space
    const int64_t c0 = cx << log2CS;                     // first position of the chunk
    const int64_t a = max(c0, p0);
    const int64_t e = min(c0 + CS, min(p0 + (r_end - r_beg), p0 + (num_rows - r_beg)));
    const int64_t lp = c0 >> log2P;
    if (a >= e || lp >= max_lp) return;
    const int32_t page = page_of[(static_cast<int64_t>(b) * hkv + g) * max_lp + lp];
    if (page < 0 || page >= num_pages) return;

    const int32_t dchunks = D / 8;
    const int32_t base = static_cast<int32_t>(c0 & (P - 1));    // slot of the chunk's first position
    const int32_t s_lo = static_cast<int32_t>(a - c0), s_hi = static_cast<int32_t>(e - c0);
    const int32_t ld = D + 8;

    // K: straight copy, one 16-byte vector per (slot, 8 dims); V rows into LDS.
    for (int32_t c = threadIdx.x; c < (s_hi - s_lo) * dchunks; c += kThreads) {
        const int32_t s = s_lo + c / dchunks, dc = c % dchunks;
        const int64_t row = r_beg + (c0 + s - p0);
        const int64_t src = (row * hkv + g) * D + dc * 8;
        const u32x4 kv = *reinterpret_cast<const u32x4 *>(k_new + src);
        *reinterpret_cast<u32x4 *>(k_pool + ((static_cast<int64_t>(page) << log2P) + base + s) * D + dc * 8) = kv;
        *reinterpret_cast<u32x4 *>(vtile + s * ld + dc * 8) = *reinterpret_cast<const u32x4 *>(v_new + src);
    }
    __syncthreads();

    // V: transposed write, 8 consecutive slots of one dimension per lane.
    u16 *vpage = v_pool + static_cast<int64_t>(page) * D * P + base;
    const int32_t schunks = CS / 8;
    for (int32_t c = threadIdx.x; c < D * schunks; c += kThreads) {
        const int32_t d = c / schunks, s8 = (c % schunks) * 8;
        if (s8 + 8 <= s_lo || s8 >= s_hi) continue;
        if (s8 >= s_lo && s8 + 8 <= s_hi) {
            u32x4 packed;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                packed[i] = static_cast<unsigned>(vtile[(s8 + 2 * i) * ld + d]) |
                            (static_cast<unsigned>(vtile[(s8 + 2 * i + 1) * ld + d]) << 16);
            *reinterpret_cast<u32x4 *>(vpage + static_cast<int64_t>(d) * P + s8) = packed;
        } else {
            for (int i = 0; i < 8; ++i) {
                const int32_t s = s8 + i;
                if (s >= s_lo && s < s_hi) vpage[static_cast<int64_t>(d) * P + s] = vtile[s * ld + d];
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void gather_pages_kernel(const int32_t *__restrict__ page_ids, int64_t n,
                                                                const u16 *__restrict__ k_pool,
                                                                const u16 *__restrict__ v_pool, int64_t num_pages,
                                                                int32_t D, int32_t log2P, u16 *__restrict__ k_out,
                                                                u16 *__restrict__ v_out)
{
    const int32_t P = 1 << log2P;
    const int64_t per_page = static_cast<int64_t>(P) * D;
    const int64_t total = n * per_page;
    for (int64_t x = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; x < total;
         x += static_cast<int64_t>(gridDim.x) * kThreads) {
        const int64_t i = x / per_page;
        const int32_t rem = static_cast<int32_t>(x % per_page);
        const int32_t slot = rem / D, d = rem % D;
        const int32_t page = page_ids[i];
        u16 kv = 0, vv = 0;
        if (page >= 0 && page < num_pages) {
            kv = k_pool[static_cast<int64_t>(page) * per_page + static_cast<int64_t>(slot) * D + d];
            vv = v_pool[static_cast<int64_t>(page) * per_page + static_cast<int64_t>(d) * P + slot];
        }
        k_out[x] = kv;
        v_out[x] = vv;
    }
}

int log2_of(int p)
{
    int l = 0;
    while ((1 << l) < p) ++l;
    return l;
}

// RoPE re-alignment (RedKnot summary page, "Elastic Sparsity": recovery starts
// by aligning reused K to its new positions). A K row encoded with rotary
// angles p * theta_i becomes the row encoded at p + delta by one more rotation
// of each pair (i, i + D/2) by delta * theta_i. One workgroup per entry (page,
// slot range, delta): the D/2 angles are reduced and evaluated in fp64 once,
// then every slot rotates in fp32 and rounds to bf16 (nearest even).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(kThreads) void rope_realign_kernel(const int32_t *__restrict__ entries, u16 *k_pool,
                                                                int64_t num_pages, int32_t D, int32_t log2P,
                                                                double log2_base)
{
    __shared__ float cs[2][64];   // cos, sin per frequency (D <= 128)
    const int32_t *ent = entries + static_cast<int64_t>(blockIdx.x) * 4;
    const int32_t page = ent[0], slot0 = ent[1], nslots = ent[2], delta = ent[3];
    const int32_t P = 1 << log2P, H = D / 2;
    if (page < 0 || page >= num_pages || slot0 < 0 || slot0 >= P || nslots <= 0) return;
    const int32_t s_end = slot0 + min(nslots, P - slot0);
    if (threadIdx.x < H) {
        const double theta = exp2(-log2_base * (2.0 * threadIdx.x / D));
        const double ang = static_cast<double>(delta) * theta;
        cs[0][threadIdx.x] = static_cast<float>(cos(ang));
        cs[1][threadIdx.x] = static_cast<float>(sin(ang));
    }
    __syncthreads();
    const int32_t per_slot = H / 8;   // threads per slot: 8 pairs each
    u16 *base = k_pool + (static_cast<int64_t>(page) << log2P) * D;
    for (int32_t c = threadIdx.x; c < (s_end - slot0) * per_slot; c += kThreads) {
        const int32_t s = slot0 + c / per_slot, i0 = (c % per_slot) * 8;
        bf16x8 *px = reinterpret_cast<bf16x8 *>(base + static_cast<int64_t>(s) * D + i0);
        bf16x8 *py = reinterpret_cast<bf16x8 *>(base + static_cast<int64_t>(s) * D + H + i0);
        const bf16x8 x = *px, y = *py;
        bf16x8 xo, yo;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float c0 = cs[0][i0 + k], s0 = cs[1][i0 + k];
            const float xf = static_cast<float>(x[k]), yf = static_cast<float>(y[k]);
            xo[k] = static_cast<__bf16>(xf * c0 - yf * s0);
            yo[k] = static_cast<__bf16>(xf * s0 + yf * c0);
        }
        *px = xo;
        *py = yo;
    }
}

int check_launch(const char *what)
{
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(SEGKV_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
    return SEGKV_OK;
}

}  // namespace

int launch_write_pages(const segkv_config &cfg, const void *k_new, const void *v_new, int64_t num_rows,
                       const int32_t *cu_rows, const int32_t *pos0, const int32_t *page_of, int32_t num_seqs,
                       int32_t max_lp, int32_t max_rows_per_seq, void *stream)
{
    const int32_t P = cfg.page_size, D = cfg.head_dim;
    const int32_t CS = P < 64 ? P : 64;
    const int64_t gx = (static_cast<int64_t>(max_rows_per_seq) + CS - 1) / CS + 1;
    const int64_t gy = static_cast<int64_t>(num_seqs) * cfg.num_kv_heads;
    if (gx > 0x7fffffff || gy > 65535) return fail(SEGKV_ERR_INVALID_ARG, "write_pages: grid too large");
    const size_t lds = static_cast<size_t>(CS) * (D + 8) * sizeof(unsigned short);
    hipLaunchKernelGGL(write_pages_kernel, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy)), dim3(kThreads),
                       lds, static_cast<hipStream_t>(stream), static_cast<const u16 *>(k_new),
                       static_cast<const u16 *>(v_new), num_rows, cu_rows, pos0, page_of, cfg.num_kv_heads, max_lp,
                       static_cast<u16 *>(cfg.k_pool), static_cast<u16 *>(cfg.v_pool), cfg.num_pages, D, log2_of(P), log2_of(CS));
    return check_launch("write_pages");
}

int launch_gather_pages(const segkv_config &cfg, const int32_t *page_ids, int64_t n, void *k_out, void *v_out,
                        void *stream)
{
    const int64_t total = n * cfg.page_size * cfg.head_dim;
    const int64_t blocks = std::min<int64_t>((total + kThreads - 1) / kThreads, 1 << 20);
    hipLaunchKernelGGL(gather_pages_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), page_ids, n, static_cast<const u16 *>(cfg.k_pool),
                       static_cast<const u16 *>(cfg.v_pool), cfg.num_pages, cfg.head_dim, log2_of(cfg.page_size),
                       static_cast<u16 *>(k_out), static_cast<u16 *>(v_out));
    return check_launch("gather_pages");
}

int launch_rope_realign(const segkv_config &cfg, const int32_t *entries, int64_t n, float rope_base, void *stream)
{
    hipLaunchKernelGGL(rope_realign_kernel, dim3(static_cast<unsigned>(n)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), entries, static_cast<u16 *>(cfg.k_pool), cfg.num_pages,
                       cfg.head_dim, log2_of(cfg.page_size), std::log2(static_cast<double>(rope_base)));
    return check_launch("rope_realign");
}

}  // namespace segkv
