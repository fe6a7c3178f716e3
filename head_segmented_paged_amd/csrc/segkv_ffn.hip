// Sparse FFN for gfx950 (RedKnot summary page, "Sparse FFN": only the tokens
// with the highest attention scores run the dense FFN, the rest take the
// residual identity path): the token choice, then the gathered SwiGLU FFN of
// the chosen tokens (bottom of the file).
//
// One workgroup per sequence picks the keep[b] new tokens with the largest
// attention mass, ties going to the lower row, and writes their row indices
// in ascending order. The threshold is found by a three-pass radix select
// on the float bit patterns (non-negative floats order like their bits):
// 11, 11 and 10 bits, an LDS histogram each; then one pass in row order
// writes the rows above the threshold and the first ties, positions from
// block-wide prefix counts (wave ballots).
#include <hip/hip_runtime.h>

#include "segkv_internal.h"

namespace segkv {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// Order key of a mass: its bits for a positive value; zero, negatives and NaN
// all map to 0 (they hold no attention).
__device__ __forceinline__ unsigned order_key(float x) { return x > 0.f ? __builtin_bit_cast(unsigned, x) : 0u; }

// Exclusive prefix count of pred over the workgroup (thread order), plus the total.
__device__ __forceinline__ unsigned block_prefix(bool pred, unsigned *wave_tot, unsigned &total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const unsigned long long m = __ballot(pred);
    const unsigned below = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wave] = __popcll(m);
    __syncthreads();
    unsigned before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        const unsigned t = wave_tot[w];
        before += w < wave ? t : 0u;
        all += t;
    }
    __syncthreads();
    total = all;
    return before + below;
}

__global__ __launch_bounds__(kSelThreads) void select_tokens_kernel(const float *__restrict__ mass,
                                                                    const int32_t *__restrict__ cu_rows,
                                                                    const int32_t *__restrict__ keep,
                                                                    const int32_t *__restrict__ cu_keep,
                                                                    int64_t total_rows, int32_t *__restrict__ rows_out)
{
    __shared__ unsigned hist[2048];
    __shared__ unsigned wave_tot[kSelWaves];
    __shared__ unsigned s_prefix, s_need;
    const int b = blockIdx.x;
    const int64_t r0 = cu_rows[b], r1 = cu_rows[b + 1];
    if (r0 < 0 || r1 < r0 || r1 > total_rows) return;
    const int64_t n = r1 - r0;
    const int64_t out0 = cu_keep[b];
    const int64_t room = static_cast<int64_t>(cu_keep[b + 1]) - out0;
    const int64_t k = min(min(static_cast<int64_t>(keep[b]), n), room);
    if (k <= 0 || out0 < 0) return;
    const float *m = mass + r0;

    // Radix select of the k-th largest key: after the passes, prefix is that
    // key and need is how many keys equal to it belong to the top k.
    unsigned prefix = 0, pmask = 0;
    if (threadIdx.x == 0) s_need = static_cast<unsigned>(k);
    const int shifts[3] = {21, 10, 0}, widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = shifts[pass], bins = 1 << widths[pass];
        for (int i = threadIdx.x; i < bins; i += kSelThreads) hist[i] = 0;
        __syncthreads();
        for (int64_t i = threadIdx.x; i < n; i += kSelThreads) {
            const unsigned key = order_key(m[i]);
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (bins - 1)], 1u);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            unsigned need = s_need, acc = 0;
            int chosen = 0;
            for (int j = bins - 1; j >= 0; --j) {
                if (acc + hist[j] >= need) {
                    chosen = j;
                    need -= acc;
                    break;
                }
                acc += hist[j];
            }
            s_need = need;
            s_prefix = prefix | (static_cast<unsigned>(chosen) << shift);
        }
        __syncthreads();
        prefix = s_prefix;
        pmask |= static_cast<unsigned>(bins - 1) << shift;
    }
    const unsigned thr = prefix, need = s_need;

    // Rows above the threshold, and the first `need` ties, in row order.
    unsigned ties_before = 0, written = 0;
    for (int64_t base = 0; base < n; base += kSelThreads) {
        const int64_t i = base + threadIdx.x;
        const unsigned key = i < n ? order_key(m[i]) : 0u;
        const bool in = i < n;
        unsigned tie_total, sel_total;
        const unsigned tie_rank = ties_before + block_prefix(in && key == thr, wave_tot, tie_total);
        const bool sel = in && (key > thr || (key == thr && tie_rank < need));
        const unsigned pos = written + block_prefix(sel, wave_tot, sel_total);
        if (sel) rows_out[out0 + pos] = static_cast<int32_t>(r0 + i);
        ties_before += tie_total;
        written += sel_total;
    }
}

}  // namespace

int launch_select_tokens(const float *mass, const int32_t *cu_rows, const int32_t *keep, const int32_t *cu_keep,
                         int32_t num_seqs, int64_t total_rows, int32_t *rows_out, void *stream)
{
    hipLaunchKernelGGL(select_tokens_kernel, dim3(static_cast<unsigned>(num_seqs)), dim3(kSelThreads), 0,
                       static_cast<hipStream_t>(stream), mass, cu_rows, keep, cu_keep, total_rows, rows_out);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(SEGKV_ERR_HIP, "select_tokens: %s", hipGetErrorString(err));
    return SEGKV_OK;
}

namespace {

// ---------------------------------------------------------------------------
// Gathered SwiGLU FFN of the chosen tokens, applied in place as a residual:
//   h[m]        = silu(Wg x[r_m]) * (Wu x[r_m])        (bf16, workspace)
//   x[r_m]     += Wd h[m]                               (bf16, rounded once)
// for the chosen rows r_m; every other row of x is left as it is (the
// residual identity path). Both products are bf16 MFMA GEMMs with K
// contiguous in both operands (weights stored [out][in]); the chosen rows are
// gathered straight from x by the DMA. Tile 128 x 128, K chunks of 64 in a
// two-stage LDS ring, four waves of 64 x 64 (2 x 2 blocks of 32 x 32).
// ---------------------------------------------------------------------------

typedef unsigned short u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kGemmThreads = 256;
constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kTileBytes = kBM * kBK * 2;   // one 128 x 64 bf16 operand tile, 16 KB
constexpr int kRowBytes = kBK * 2;          // 128 B per tile row

// Row r of a tile keeps its 16-byte chunk c at position c ^ gswz(r).
__device__ __forceinline__ int gswz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ void gdma16(__amdgpu_buffer_rsrc_t rsrc, char *lds, unsigned voffset, unsigned soffset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)lds, 16, voffset, soffset, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const u16 *base, int64_t bytes)
{
    const int64_t n = bytes < 0xffffffffll ? bytes : 0xffffffffll;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<u16 *>(base), 0, static_cast<int>(static_cast<uint32_t>(n)),
                                             0x00020000);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __builtin_amdgcn_exp2f(-g * 1.44269504088896340736f)); }

// GATE: A = x rows chosen by rows[], B0 = Wg, B1 = Wu -> h. Otherwise A = h,
// B0 = Wd -> x[rows[m]] += result.
template <bool GATE>
__global__ __launch_bounds__(kGemmThreads, 1) void ffn_gemm_kernel(
    const u16 *__restrict__ a, int64_t a_bytes, const int32_t *__restrict__ rows, int64_t x_rows, int32_t M,
    int32_t K, const u16 *__restrict__ b0, const u16 *__restrict__ b1, int64_t b_bytes, int32_t N,
    u16 *__restrict__ out)
{
    constexpr int kTiles = GATE ? 3 : 2;                  // A, B0 (, B1)
    __shared__ __attribute__((aligned(1024))) char st0[kTiles * kTileBytes];
    __shared__ __attribute__((aligned(1024))) char st1[kTiles * kTileBytes];

    const int n0 = blockIdx.x * kBN, m0 = blockIdx.y * kBM;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const int wm = wave & 1, wn = wave >> 1;

    // DMA: each wave moves 4 KB of every tile per K chunk, 16 bytes a lane.
    const __amdgpu_buffer_rsrc_t ra = gemm_rsrc(a, a_bytes), rb0 = gemm_rsrc(b0, b_bytes);
    const __amdgpu_buffer_rsrc_t rb1 = gemm_rsrc(GATE ? b1 : b0, b_bytes);
    unsigned aoff[4], boff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = (wave * 4 + i) * 1024 + lane * 16;
        const int r = p / kRowBytes, c = ((p % kRowBytes) / 16) ^ gswz(r);
        const int m = m0 + r;
        int64_t arow = -1;
        if (m < M) arow = GATE ? rows[m] : m;
        // A row missing (past M, or a chosen row outside x): read row 0 instead;
        // only output rows that are never written depend on it.
        if (arow < 0 || (GATE && arow >= x_rows)) arow = 0;
        aoff[i] = static_cast<unsigned>(arow * K * 2 + c * 16);
        boff[i] = static_cast<unsigned>(static_cast<int64_t>(n0 + r) * K * 2 + c * 16);
    }
    auto dma = [&](char *stage, int k0) {
        const unsigned so = static_cast<unsigned>(k0 * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            char *dst = stage + (wave * 4 + i) * 1024;
            gdma16(ra, dst, aoff[i], so);
            gdma16(rb0, dst + kTileBytes, boff[i], so);
            if constexpr (GATE) gdma16(rb1, dst + 2 * kTileBytes, boff[i], so);
        }
    };

    // Operand addresses: A rows wm*64 + 32 bi + col, B rows wn*64 + 32 bj + col.
    unsigned arow_lds[2], brow_lds[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        arow_lds[i] = static_cast<unsigned>((wm * 64 + 32 * i + col) * kRowBytes);
        brow_lds[i] = static_cast<unsigned>((wn * 64 + 32 * i + col) * kRowBytes);
    }
    const int aswz[2] = {gswz(wm * 64 + col), gswz(wm * 64 + 32 + col)};
    const int bswz[2] = {gswz(wn * 64 + col), gswz(wn * 64 + 32 + col)};

    f32x16 acc0[2][2], acc1[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            acc0[i][j] = f32x16{};
            acc1[i][j] = f32x16{};
        }

    auto compute = [&](const char *stage) {
#pragma unroll
        for (int s = 0; s < kBK / 16; ++s) {
            bf16x8 av[2], bv[2], cv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                av[i] = *reinterpret_cast<const bf16x8 *>(stage + arow_lds[i] + (((2 * s + half) ^ aswz[i]) << 4));
                bv[i] = *reinterpret_cast<const bf16x8 *>(stage + kTileBytes + brow_lds[i] +
                                                          (((2 * s + half) ^ bswz[i]) << 4));
                if constexpr (GATE)
                    cv[i] = *reinterpret_cast<const bf16x8 *>(stage + 2 * kTileBytes + brow_lds[i] +
                                                              (((2 * s + half) ^ bswz[i]) << 4));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    acc0[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc0[i][j], 0, 0, 0);
                    if constexpr (GATE)
                        acc1[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], cv[j], acc1[i][j], 0, 0, 0);
                }
        }
    };

    const int chunks = K / kBK;
    dma(st0, 0);
    __syncthreads();
    int kc = 0;
    for (; kc + 1 < chunks; kc += 2) {
        dma(st1, (kc + 1) * kBK);
        compute(st0);
        __syncthreads();
        if (kc + 2 < chunks) dma(st0, (kc + 2) * kBK);
        compute(st1);
        __syncthreads();
    }
    if (kc < chunks) compute(st0);

    // Epilogue: lane holds column n, registers rows 8 (e / 4) + 4 half + e % 4.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + wn * 64 + 32 * j + col;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + wm * 64 + 32 * i + 8 * (e >> 2) + 4 * half + (e & 3);
                if (m >= M) continue;
                if constexpr (GATE) {
                    const __bf16 hv = static_cast<__bf16>(silu(acc0[i][j][e]) * acc1[i][j][e]);
                    out[static_cast<int64_t>(m) * N + n] = __builtin_bit_cast(u16, hv);
                } else {
                    const int64_t r = rows[m];
                    if (r < 0 || r >= x_rows) continue;
                    u16 *px = out + r * N + n;
                    const float xv = static_cast<float>(__builtin_bit_cast(__bf16, *px));
                    *px = __builtin_bit_cast(u16, static_cast<__bf16>(xv + acc0[i][j][e]));
                }
            }
        }
}

}  // namespace

int launch_sparse_ffn(void *x, int64_t x_rows, int32_t d_model, int32_t d_ff, const int32_t *sel_rows,
                      int32_t n_sel, const void *w_gate, const void *w_up, const void *w_down, void *h, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    const unsigned mt = static_cast<unsigned>((n_sel + kBM - 1) / kBM);
    const int64_t x_bytes = x_rows * d_model * 2, w_bytes = static_cast<int64_t>(d_ff) * d_model * 2;
    hipLaunchKernelGGL((ffn_gemm_kernel<true>), dim3(static_cast<unsigned>(d_ff / kBN), mt), dim3(kGemmThreads), 0,
                       s, static_cast<const u16 *>(x), x_bytes, sel_rows, x_rows, n_sel, d_model,
                       static_cast<const u16 *>(w_gate), static_cast<const u16 *>(w_up), w_bytes, d_ff,
                       static_cast<u16 *>(h));
    hipLaunchKernelGGL((ffn_gemm_kernel<false>), dim3(static_cast<unsigned>(d_model / kBN), mt), dim3(kGemmThreads),
                       0, s, static_cast<const u16 *>(h), static_cast<int64_t>(n_sel) * d_ff * 2, sel_rows, x_rows,
                       n_sel, d_ff, static_cast<const u16 *>(w_down), static_cast<const u16 *>(nullptr), w_bytes,
                       d_model, static_cast<u16 *>(x));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(SEGKV_ERR_HIP, "sparse_ffn: %s", hipGetErrorString(err));
    return SEGKV_OK;
}

}  // namespace segkv
