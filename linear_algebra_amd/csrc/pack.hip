// Triangular pack / unpack between per-layer d x d float32 matrices and one
// fused float32 buffer holding their upper triangles (incl. the diagonal),
// row by row, layers back to back.  Both directions are bit-exact copies.
//
// Pack walks the fused buffer in chunks that never cross a factor: the
// workgroup finds its factor once, and lanes take consecutive packed
// elements, so reads run along matrix rows and writes are contiguous.  The
// row of a packed index comes from the closed-form row start i*d - i*(i-1)/2.
//
// Unpack works on 64 x 64 tiles of the upper block triangle of each matrix:
// the tile's rows are read from the fused buffer (contiguous runs), staged in
// LDS, and written both to their own place and, transposed through LDS, to
// the mirrored tile, so every global write is a coalesced row segment.
#include "device_common.h"
#include "internal.h"

namespace kfac {
namespace {

constexpr int PT = 256;
constexpr int PACK_PER = kPackChunk / PT;  // packed elements per thread
constexpr int PACK_CHUNK = kPackChunk;

__device__ __forceinline__ int find_layer(const PackLayer* L, int n, int64_t p, bool by_tile) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        const int64_t b = by_tile ? L[mid].tile_begin : L[mid].off;
        if (b <= p) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ int64_t row_start(int64_t i, int64_t d) { return i * d - i * (i - 1) / 2; }

// Row of the upper triangle holding local packed index q.
__device__ __forceinline__ int64_t row_of(int64_t q, int64_t d) {
    const double a = 2.0 * (double)d + 1.0;
    int64_t i = (int64_t)((a - sqrt(a * a - 8.0 * (double)q)) * 0.5);
    if (i < 0) i = 0;
    if (i > d - 1) i = d - 1;
    while (i > 0 && row_start(i, d) > q) --i;
    while (i + 1 < d && row_start(i + 1, d) <= q) ++i;
    return i;
}

// Row of the upper triangle of a d x d matrix holding local packed index q
// (row i starts at i*d - i*(i-1)/2).  An fp32 square root lands within one
// row of the answer for d <= 16384; integer checks settle it.
__device__ __forceinline__ int64_t row_of_fast(int64_t q, int64_t d) {
    const float a = 2.0f * (float)d + 1.0f;
    int64_t i = (int64_t)((a - sqrtf(fmaxf(a * a - 8.0f * (float)q, 0.0f))) * 0.5f);
    i = i < 0 ? 0 : (i > d - 1 ? d - 1 : i);
    while (i > 0 && row_start(i, d) > q) --i;
    while (i + 1 < d && row_start(i + 1, d) <= q) ++i;
    return i;
}

// One workgroup copies PACK_CHUNK consecutive packed elements of a single
// factor; thread t takes elements t + PT*s, so every wave instruction reads
// a run of one matrix row and writes 256 contiguous bytes.
__global__ __launch_bounds__(PT) void pack_kernel(const PackLayer* __restrict__ layers, int n,
                                                  float* __restrict__ packed, int64_t blocks) {
    const int64_t blk = blockIdx.x;
    if (blk >= blocks) return;
    const PackLayer L = layers[find_layer(layers, n, blk, true)];
    const int64_t d = L.d;
    const int64_t total = d * (d + 1) / 2;
    const int64_t q0 = (blk - L.tile_begin) * PACK_CHUNK;
    // row of the first element from the closed form, later ones by walking
    // forward (the next element is PT further on, at most a few rows down)
    float v[PACK_PER];
    int64_t q = q0 + threadIdx.x;
    int64_t i = row_of_fast(q < total ? q : total - 1, d);
    int64_t rs = row_start(i, d), re = rs + (d - i);   // [rs, re) are row i's packed indices
#pragma unroll
    for (int s = 0; s < PACK_PER; ++s, q += PT) {
        if (q < total) {
            while (q >= re) {
                ++i;
                rs = re;
                re += d - i;
            }
            v[s] = L.m[i * d + i + (q - rs)];
        }
    }
#pragma unroll
    for (int s = 0; s < PACK_PER; ++s) {
        const int64_t q = q0 + threadIdx.x + PT * s;
        if (q < total) packed[L.off + q] = v[s];
    }
}

constexpr int UT = kUnpackTile;

__global__ __launch_bounds__(PT) void unpack_kernel(const PackLayer* __restrict__ layers, int n,
                                                    const float* __restrict__ packed, int64_t tiles) {
    __shared__ float S[UT][UT + 1];
    const int64_t tile = xcd_remap(blockIdx.x, gridDim.x);
    if (tile >= tiles) return;
    const PackLayer L = layers[find_layer(layers, n, tile, true)];
    int ti, tj;
    upper_decode(tile - L.tile_begin, L.tiles_1d, ti, tj);
    const int64_t d = L.d;
    const int64_t r0 = (int64_t)ti * UT, c0 = (int64_t)tj * UT;
    const float* src = packed + L.off;

    // stage the tile's upper entries (i <= j) from the fused buffer: thread
    // t handles rows t/64 + 4s, column t%64, all loads in flight together
    constexpr int PERT = UT * UT / PT;
    const int q0 = threadIdx.x / UT, l = threadIdx.x % UT;
    float v[PERT];
#pragma unroll
    for (int s = 0; s < PERT; ++s) {
        const int64_t i = r0 + q0 + 4 * s, j = c0 + l;
        v[s] = (i < d && j < d && j >= i) ? src[row_start(i, d) + (j - i)] : 0.0f;
    }
#pragma unroll
    for (int s = 0; s < PERT; ++s) S[q0 + 4 * s][l] = v[s];
    __syncthreads();

    // the tile itself: on diagonal tiles the lower half is the mirror
#pragma unroll
    for (int s = 0; s < PERT; ++s) {
        const int r = q0 + 4 * s, c = l;
        const int64_t i = r0 + r, j = c0 + c;
        if (i < d && j < d) L.m[i * d + j] = (j >= i) ? S[r][c] : S[c][r];
    }
    // the mirrored tile below the diagonal, written row by row
    if (ti != tj) {
#pragma unroll
        for (int s = 0; s < PERT; ++s) {
            const int c = q0 + 4 * s, r = l;   // destination row c0+c, column r0+r
            const int64_t i = c0 + c, j = r0 + r;
            if (i < d && j < d) L.m[i * d + j] = S[r][c];
        }
    }
}

}  // namespace

hipError_t launch_pack(const PackLayer* layers_dev, int n, float* packed, int64_t blocks, hipStream_t stream) {
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(PT), 0, stream, layers_dev, n, packed, blocks);
    return hipGetLastError();
}

hipError_t launch_unpack(const PackLayer* layers_dev, int n, const float* packed, int64_t tiles,
                         hipStream_t stream) {
    if (tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)tiles), dim3(PT), 0, stream, layers_dev, n, packed, tiles);
    return hipGetLastError();
}

}  // namespace kfac
