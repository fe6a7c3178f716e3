// Sparse FFN token selection for gfx950 (RedKnot summary page, "Sparse
// FFN": only the tokens with the highest attention scores run the dense
// FFN, the rest take the residual identity path).
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

}  // namespace segkv
