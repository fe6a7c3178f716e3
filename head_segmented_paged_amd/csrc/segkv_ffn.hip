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
// gathered straight from x by the DMA. Tile 256 x 128 (for the first product
// the gate and the up projection of it), K slices of 64 in an LDS ring, eight
// waves of 64 x 64 (2 x 2 blocks of 32 x 32; for the first product also the
// up projection's 2 x 2).
// ---------------------------------------------------------------------------

typedef unsigned short u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kGemmThreads = 512;                 // eight waves, two per SIMD
constexpr int kBM = 256;                    // A rows (chosen tokens) per tile
constexpr int kBN = 128;                    // output columns per tile

// Row r of a tile of BK-wide rows keeps its 16-byte chunk c at position
// c ^ gswz<BK>(r): sixteen lanes reading one chunk of sixteen consecutive rows
// hit sixteen distinct 16-byte bank groups (64-byte rows: four rows per
// 256-byte bank line, four chunk positions; 128-byte rows: two and eight).
template <int BK>
__device__ __forceinline__ int gswz(int r) { return BK == 32 ? (r >> 2) & 3 : (r >> 1) & 7; }

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

// Wait until at most N of this wave's vector-memory operations (here: LDS
// DMAs) are outstanding and all its LDS reads are done, then meet the other
// waves. Unlike __syncthreads, which waits for every DMA, this leaves the
// newer stages in flight.
template <int N>
__device__ __forceinline__ void wait_dma_barrier()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // The empty asm statements are compiler memory barriers: no load or store
    // of shared memory moves across the wait and the barrier.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __builtin_amdgcn_exp2f(-g * 1.44269504088896340736f)); }

// GATE: A = x rows chosen by rows[], B0 = Wg, B1 = Wu -> h. Otherwise A = h,
// B0 = Wd -> x[rows[m]] += result.
// A workgroup computes a 256 x 128 output tile (for GATE both the gate and the
// up projection of it), eight waves of 64 x 64 each, two per SIMD. The tile
// size sets how many bytes each MFMA needs from L2: 128 flops per byte staged
// into LDS here, against 64-85 for 128 x 128 tiles. Operands stream through an
// LDS ring of 64-wide K slices, all but one in flight while one is multiplied.
template <bool GATE>
__global__ __launch_bounds__(kGemmThreads, 1) void ffn_gemm_kernel(
    const u16 *__restrict__ a, int64_t a_bytes, const int32_t *__restrict__ rows, int64_t x_rows, int32_t M,
    int32_t K, const u16 *__restrict__ b0, const u16 *__restrict__ b1, int64_t b_bytes, int32_t N,
    u16 *__restrict__ out)
{
    // K per stage: 64 (each stage's barrier is amortised over 2048 MFMA cycles
    // per SIMD for GATE, 1024 for the down projection; 32-wide slices in
    // deeper rings measured 4-7 % slower).
    constexpr int kBK = 64;
    constexpr int kRowBytes = kBK * 2;
    constexpr int kATileBytes = kBM * kRowBytes;
    constexpr int kBRows = GATE ? 2 * kBN : kBN;           // B tile rows: gate rows then up rows, or down rows
    constexpr int kBTileBytes = kBRows * kRowBytes;
    constexpr int kStage = kATileBytes + kBTileBytes;      // 32 KB or 48 KB
    constexpr int kAInstr = kATileBytes / 1024 / 8;        // DMA instructions per wave and stage
    constexpr int kBInstr = kBTileBytes / 1024 / 8;
    constexpr int kInstr = kAInstr + kBInstr;
    constexpr int kBCols = GATE ? 4 : 2;                   // 32-column B blocks per wave (gate 0, 1; up 2, 3)
    // LDS ring of kStages stages (2 x 64 KB and 3 x 48 KB), indexed by
    // constants only, so the compiler sees that a DMA into one stage does not
    // alias the LDS reads of another and adds no wait for it.
    constexpr int kStages = GATE ? 2 : 3;
    __shared__ __attribute__((aligned(1024))) char ring[kStages][kStage];

    const int m0 = blockIdx.x * kBM, n0 = blockIdx.y * kBN;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const int wm = wave & 3, wn = wave >> 2;

    // DMA: every wave moves kInstr KB of each stage, 16 bytes a lane. A B-tile
    // instruction covers 16 rows, all of one weight matrix: for GATE waves
    // 0-3 fill the gate rows and waves 4-7 the up rows.
    const __amdgpu_buffer_rsrc_t ra = gemm_rsrc(a, a_bytes);
    const __amdgpu_buffer_rsrc_t rb = gemm_rsrc(GATE && wave >= 4 ? b1 : b0, b_bytes);
    const __amdgpu_buffer_rsrc_t rnone = gemm_rsrc(a, 0);   // empty range: the ring's tail DMAs read nothing
    unsigned aoff[kAInstr], boff[kBInstr];
#pragma unroll
    for (int i = 0; i < kAInstr; ++i) {
        const int p = (wave * kAInstr + i) * 1024 + lane * 16;
        const int r = p / kRowBytes, c = ((p % kRowBytes) / 16) ^ gswz<kBK>(r);
        const int m = m0 + r;
        int64_t arow = -1;
        if (m < M) arow = GATE ? rows[m] : m;
        // A row missing (past M, or a chosen row outside x): read row 0 instead;
        // only output rows that are never written depend on it.
        if (arow < 0 || (GATE && arow >= x_rows)) arow = 0;
        aoff[i] = static_cast<unsigned>(arow * K * 2 + c * 16);
    }
#pragma unroll
    for (int i = 0; i < kBInstr; ++i) {
        const int p = (wave * kBInstr + i) * 1024 + lane * 16;
        const int r = p / kRowBytes, c = ((p % kRowBytes) / 16) ^ gswz<kBK>(r);
        const int wrow = n0 + (r % kBN);
        boff[i] = static_cast<unsigned>(static_cast<int64_t>(wrow) * K * 2 + c * 16);
    }
    // Stage kc of the K loop; past the end the same count of DMAs reads an
    // empty range (zeros into a stage nobody reads), so every wait below
    // counts the same instructions.
    const int chunks = K / kBK;
    auto dma = [&](char *stage, int kc) {
        const bool live = kc < chunks;
        const unsigned so = live ? static_cast<unsigned>(kc * kBK * 2) : 0u;
#pragma unroll
        for (int i = 0; i < kAInstr; ++i) gdma16(live ? ra : rnone, stage + (wave * kAInstr + i) * 1024, aoff[i], so);
#pragma unroll
        for (int i = 0; i < kBInstr; ++i)
            gdma16(live ? rb : rnone, stage + kATileBytes + (wave * kBInstr + i) * 1024, boff[i], so);
    };

    // Operand rows: A rows wm * 64 + 32 i + col; B rows wn * 64 + 32 j + col
    // (and the same plus kBN for the up rows).
    unsigned arow_lds[2], brow_lds[kBCols];
    int aswz[2], bswz[kBCols];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + 32 * i + col;
        arow_lds[i] = static_cast<unsigned>(r * kRowBytes);
        aswz[i] = gswz<kBK>(r);
    }
#pragma unroll
    for (int j = 0; j < kBCols; ++j) {
        const int r = (j >> 1) * kBN + wn * 64 + 32 * (j & 1) + col;
        brow_lds[j] = static_cast<unsigned>(kATileBytes + r * kRowBytes);
        bswz[j] = gswz<kBK>(r);
    }

    f32x16 acc[2][kBCols];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < kBCols; ++j) acc[i][j] = f32x16{};

    struct Ops {
        bf16x8 a[2], b[kBCols];
    };
    auto load_ops = [&](Ops &op, const char *stage, int s) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            op.a[i] = *reinterpret_cast<const bf16x8 *>(stage + arow_lds[i] + (((2 * s + half) ^ aswz[i]) << 4));
#pragma unroll
        for (int j = 0; j < kBCols; ++j)
            op.b[j] = *reinterpret_cast<const bf16x8 *>(stage + brow_lds[j] + (((2 * s + half) ^ bswz[j]) << 4));
    };
    auto mfmas = [&](const Ops &op) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < kBCols; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op.a[i], op.b[j], acc[i][j], 0, 0, 0);
    };
    // Each k-step's operands are read while the previous k-step's MFMAs run:
    // the scheduling groups put one LDS read after each of the first MFMAs of
    // a step (the compiler would otherwise read each step's operands right
    // before its MFMAs and leave the matrix core idle for the LDS latency).
    constexpr int kKSteps = kBK / 16;
    auto compute = [&](const char *stage) {
        Ops x, y;
        load_ops(x, stage, 0);
#pragma unroll
        for (int s = 0; s < kKSteps; s += 2) {
            load_ops(y, stage, s + 1);
            mfmas(x);
            if (s + 2 < kKSteps) load_ops(x, stage, s + 2);
            mfmas(y);
        }
        constexpr int kReads = 2 + kBCols, kMfma = 2 * kBCols;
        __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
#pragma unroll
        for (int st = 0; st + 1 < kKSteps; ++st) {
#pragma unroll
            for (int r = 0; r < kReads; ++r) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kReads, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kMfma, 0);
    };
    // Stage kc: wait for its DMA (the newer stages stay in flight), refill the
    // stage used one step earlier with stage kc + kStages - 1, multiply stage kc.
    auto step = [&](const char *cur, char *refill, int kc) {
        wait_dma_barrier<(kStages - 2) * kInstr>();
        dma(refill, kc + kStages - 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(cur);
    };

    // Rounded up to whole laps of the ring: the extra stages are zeros.
#pragma unroll
    for (int i = 0; i + 1 < kStages; ++i) dma(ring[i], i);
    for (int kc = 0; kc < chunks; kc += kStages) {
#pragma unroll
        for (int i = 0; i < kStages; ++i) step(ring[i], ring[(i + kStages - 1) % kStages], kc + i);
    }
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0): no DMA outlives the loop

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
                    const __bf16 hv = static_cast<__bf16>(silu(acc[i][j][e]) * acc[i][j + 2][e]);
                    out[static_cast<int64_t>(m) * N + n] = __builtin_bit_cast(u16, hv);
                } else {
                    const int64_t r = rows[m];
                    if (r < 0 || r >= x_rows) continue;
                    u16 *px = out + r * N + n;
                    const float xv = static_cast<float>(__builtin_bit_cast(__bf16, *px));
                    *px = __builtin_bit_cast(u16, static_cast<__bf16>(xv + acc[i][j][e]));
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
    hipLaunchKernelGGL((ffn_gemm_kernel<true>), dim3(mt, static_cast<unsigned>(d_ff / kBN)), dim3(kGemmThreads), 0,
                       s, static_cast<const u16 *>(x), x_bytes, sel_rows, x_rows, n_sel, d_model,
                       static_cast<const u16 *>(w_gate), static_cast<const u16 *>(w_up), w_bytes, d_ff,
                       static_cast<u16 *>(h));
    hipLaunchKernelGGL((ffn_gemm_kernel<false>), dim3(mt, static_cast<unsigned>(d_model / kBN)), dim3(kGemmThreads),
                       0, s, static_cast<const u16 *>(h), static_cast<int64_t>(n_sel) * d_ff * 2, sel_rows, x_rows,
                       n_sel, d_ff, static_cast<const u16 *>(w_down), static_cast<const u16 *>(nullptr), w_bytes,
                       d_model, static_cast<u16 *>(x));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(SEGKV_ERR_HIP, "sparse_ffn: %s", hipGetErrorString(err));
    return SEGKV_OK;
}

}  // namespace segkv
