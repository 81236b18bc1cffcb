// Triangular pack / unpack between per-layer d x d float32 matrices and one
// fused float32 buffer holding their upper triangles (incl. the diagonal),
// row by row, layers back to back.  Both directions are bit-exact copies.
//
// Pack walks the fused buffer: each thread owns 4 consecutive packed
// elements, so the writes are aligned 16-byte stores that tile the buffer
// without gaps, and consecutive threads read consecutive entries of the same
// matrix row.  The (layer, row, column) of a packed index comes from a
// binary search over the layer offsets and the closed-form row start
// i*d - i*(i-1)/2.
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
constexpr int PER = 4;  // packed elements per thread

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

__global__ __launch_bounds__(PT) void pack_kernel(const PackLayer* __restrict__ layers, int n,
                                                  float* __restrict__ packed, int64_t total) {
    const int64_t g = (int64_t)blockIdx.x * PT + threadIdx.x;
    const int64_t p0 = g * PER;
    if (p0 >= total) return;

    int l = find_layer(layers, n, p0, false);
    PackLayer L = layers[l];
    int64_t q = p0 - L.off;
    int64_t i = row_of(q, L.d);
    int64_t j = i + (q - row_start(i, L.d));

    float v[PER];
#pragma unroll
    for (int s = 0; s < PER; ++s) {
        if (p0 + s < total) {
            // a layer ends exactly where the next begins; skip empty ones
            while (p0 + s >= L.off + L.d * (L.d + 1) / 2) {
                L = layers[++l];
                i = 0;
                j = 0;
            }
            v[s] = L.m[i * L.d + j];
            if (++j == L.d) { ++i; j = i; }
        } else {
            v[s] = 0.0f;
        }
    }
    if (p0 + PER <= total && ((reinterpret_cast<uintptr_t>(packed + p0) & 15) == 0)) {
        *reinterpret_cast<float4*>(packed + p0) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
        for (int s = 0; s < PER; ++s)
            if (p0 + s < total) packed[p0 + s] = v[s];
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

hipError_t launch_pack(const PackLayer* layers_dev, int n, float* packed, int64_t total, hipStream_t stream) {
    if (total <= 0) return hipSuccess;
    const int64_t threads = ceil_div(total, PER);
    const int64_t blocks = ceil_div(threads, PT);
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(PT), 0, stream, layers_dev, n, packed, total);
    return hipGetLastError();
}

hipError_t launch_unpack(const PackLayer* layers_dev, int n, const float* packed, int64_t tiles,
                         hipStream_t stream) {
    if (tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)tiles), dim3(PT), 0, stream, layers_dev, n, packed, tiles);
    return hipGetLastError();
}

}  // namespace kfac
