// fp32 MFMA GEMM for the factor (syrk, upper tiles, running average) and
// precondition (two plain products) stages.
//
// C = alpha * Aop^T Bop, Aop [K][lda], Bop [K][ldb], both with the reduction
// index as the slow (row) index, so every staged K-slab is a set of
// contiguous row segments and the global loads coalesce.
//
// Tile 128 x 128 per workgroup of 4 waves (2 x 2, 64 x 64 each, four
// v_mfma_f32_32x32x2f32 accumulators per wave).  K is staged through two LDS
// buffers of 16 rows per operand; the next slab is fetched into registers
// while the current one feeds the matrix cores.  Products are summed in
// float32 over sub-chunks of kGemmSubK rows and then folded into a second
// float32 sum, which keeps the rounding error of long reductions (hundreds of
// thousands of rows) near that of a 512-term sum.
#include "device_common.h"
#include "internal.h"

namespace kfac {
namespace {

constexpr int BM = kGemmTile;
constexpr int BK = kGemmBK;
constexpr int NT = kGemmThreads;
constexpr int LOADS = BK * BM / NT;  // elements of one operand slab per thread (8)
constexpr int SUB_STAGES = kGemmSubK / BK;

template <bool BF16>
__device__ __forceinline__ float load_op(const void* base, int64_t idx) {
    if constexpr (BF16) {
        return bf16_to_f32(static_cast<const uint16_t*>(base)[idx]);
    } else {
        return static_cast<const float*>(base)[idx];
    }
}

__device__ __forceinline__ int find_prob(const GemmProb* probs, int nprob, int64_t item, bool reduce) {
    int lo = 0, hi = nprob - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        const int64_t begin = reduce ? probs[mid].red_begin : probs[mid].item_begin;
        if (begin <= item) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Epilogue for one output element (row i, column j of the problem).
__device__ __forceinline__ void store_elem(const GemmProb& P, int i, int j, float v, float eps, int first) {
    if (i >= P.M || j >= P.N) return;
    if (P.mode == kModeFactor) {
        if (j < i) return;
        const float f = v * P.alpha;
        float* dst = P.c + (int64_t)i * P.ldc + j;
        *dst = first ? f : eps * (*dst) + (1.0f - eps) * f;
    } else {
        P.c[(int64_t)i * P.ldc + j] = v * P.alpha;
    }
}

template <bool BF16>
__global__ __launch_bounds__(NT, 2) void gemm_tn_kernel(GemmLaunch L, int64_t items) {
    __shared__ float As[2][BK][BM];
    __shared__ float Bs[2][BK][BM];

    const int64_t item = xcd_remap(blockIdx.x, gridDim.x);
    if (item >= items) return;
    const GemmProb P = L.probs[find_prob(L.probs, L.nprob, item, false)];

    const int64_t w = item - P.item_begin;
    const int kc = (int)(w / P.ntiles);
    const int t = (int)(w % P.ntiles);
    int ti, tj;
    if (P.mode == kModeFactor) {
        upper_decode(t, P.tiles_m, ti, tj);
    } else {
        ti = t / P.tiles_n;
        tj = t % P.tiles_n;
    }
    const int m0 = ti * BM, n0 = tj * BM;
    const int k_begin = kc * P.kchunk;
    const int k_end = min(P.K, k_begin + P.kchunk);
    // Factor tiles on the diagonal read the same columns for both operands.
    const bool same = (P.a == P.b) && (m0 == n0);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // the wave below the diagonal of a diagonal factor tile has nothing to compute
    const bool active = !(P.mode == kModeFactor && ti == tj && wm > wn);

    const int lc = tid & (BM - 1);  // column loaded by this thread
    const int lr = tid >> 7;        // first slab row loaded by this thread (0 or 1)

    float ra[LOADS], rb[LOADS];
    auto gload = [&](int k0) {
#pragma unroll
        for (int s = 0; s < LOADS; ++s) {
            const int row = k0 + lr + 2 * s;
            const bool rok = row < k_end;
            ra[s] = (rok && m0 + lc < P.M) ? load_op<BF16>(P.a, (int64_t)row * P.lda + m0 + lc) : 0.0f;
            if (!same) rb[s] = (rok && n0 + lc < P.N) ? load_op<BF16>(P.b, (int64_t)row * P.ldb + n0 + lc) : 0.0f;
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int s = 0; s < LOADS; ++s) {
            As[buf][lr + 2 * s][lc] = ra[s];
            if (!same) Bs[buf][lr + 2 * s][lc] = rb[s];
        }
    };

    floatx16 acc[2][2], sum[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) { acc[a][b][r] = 0.0f; sum[a][b][r] = 0.0f; }

    const int nstages = (k_end - k_begin + BK - 1) / BK;
    if (nstages > 0) {
        gload(k_begin);
        sstore(0);
    }
    __syncthreads();

    const int col_a = wm * 64 + (lane & 31);
    const int col_b = wn * 64 + (lane & 31);
    const int khalf = lane >> 5;

    for (int st = 0; st < nstages; ++st) {
        const int buf = st & 1;
        if (st + 1 < nstages) gload(k_begin + (st + 1) * BK);
        if (active) {
            const float(*Bsrc)[BM] = same ? As[buf] : Bs[buf];
#pragma unroll
            for (int ks = 0; ks < BK; ks += 2) {
                const int kk = ks + khalf;
                const float a0 = As[buf][kk][col_a];
                const float a1 = As[buf][kk][col_a + 32];
                const float b0 = Bsrc[kk][col_b];
                const float b1 = Bsrc[kk][col_b + 32];
                acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
                acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
                acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
                acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
            }
            if ((st + 1) % SUB_STAGES == 0 || st + 1 == nstages) {
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        sum[a][b] += acc[a][b];
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
                    }
            }
        }
        if (st + 1 < nstages) sstore(buf ^ 1);
        __syncthreads();
    }

    // Output layout of a 32 x 32 MFMA block: lane l holds column (l % 32);
    // register r holds row 8*(r/4) + 4*(l/32) + (r%4).
    const int ksplit = P.ksplit;
    float* part = (ksplit > 1) ? P.part + ((int64_t)kc * P.ntiles + t) * (BM * BM) : nullptr;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * 64 + a * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
                const int col = wn * 64 + b * 32 + (lane & 31);
                if (part) {
                    part[row * BM + col] = sum[a][b][r];
                } else {
                    store_elem(P, m0 + row, n0 + col, sum[a][b][r], L.eps, L.first_step);
                }
            }
}

// Sums the split-K partial tiles in chunk order and applies the epilogue.
__global__ __launch_bounds__(NT) void gemm_reduce_kernel(GemmLaunch L, int64_t tiles) {
    const int64_t tile = blockIdx.x;
    if (tile >= tiles) return;
    const GemmProb P = L.probs[find_prob(L.probs, L.nprob, tile, true)];
    const int t = (int)(tile - P.red_begin);
    int ti, tj;
    if (P.mode == kModeFactor) {
        upper_decode(t, P.tiles_m, ti, tj);
    } else {
        ti = t / P.tiles_n;
        tj = t % P.tiles_n;
    }
    // thread t sums elements t + s*NT of the tile over the K chunks in
    // chunk order; the PERR loads of one chunk are in flight together
    constexpr int PERR = BM * BM / NT;
    const int64_t stride = (int64_t)P.ntiles * (BM * BM);
    const float* base = P.part + (int64_t)t * (BM * BM);
    float s[PERR];
#pragma unroll
    for (int q = 0; q < PERR; ++q) s[q] = 0.0f;
    for (int k = 0; k < P.ksplit; ++k) {
        const float* pk = base + k * stride;
#pragma unroll
        for (int q = 0; q < PERR; ++q) s[q] += pk[threadIdx.x + q * NT];
    }
#pragma unroll
    for (int q = 0; q < PERR; ++q) {
        const int e = threadIdx.x + q * NT;
        const int row = e / BM, col = e % BM;
        store_elem(P, ti * BM + row, tj * BM + col, s[q], L.eps, L.first_step);
    }
}

}  // namespace

hipError_t launch_gemm(const GemmLaunch& L, int64_t items, hipStream_t stream, bool bf16) {
    if (items <= 0) return hipSuccess;
    if (bf16) {
        hipLaunchKernelGGL(gemm_tn_kernel<true>, dim3((unsigned)items), dim3(NT), 0, stream, L, items);
    } else {
        hipLaunchKernelGGL(gemm_tn_kernel<false>, dim3((unsigned)items), dim3(NT), 0, stream, L, items);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_reduce(const GemmLaunch& L, int64_t tiles, hipStream_t stream) {
    if (tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)tiles), dim3(NT), 0, stream, L, tiles);
    return hipGetLastError();
}

}  // namespace kfac
