// Factor inputs of real layers (kfac_im2col, kfac_grad_rows) and the
// weight/bias gradient matrix of a layer (kfac_grad_matrix).  All three move
// data only (plus one scaling), so they are bound by HBM: every kernel reads
// and writes along rows of 64 consecutive elements per wave.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace kfac {
namespace {

constexpr int NT = 256;
constexpr int T = kLayerTile;

// Layer of a work item: the last layer whose first item is <= item.
template <typename L>
__device__ __forceinline__ int find_layer(const L* layers, int n, int64_t item, int64_t L::*begin) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (layers[mid].*begin <= item) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);   // NaN stays NaN
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// One 64 x 64 tile of a[l]: lane group tx = column, rows 64 tr + ty + 4 s.
// A thread decodes its column (channel and kernel tap) once and steps its
// rows (sample, output y, output x) incrementally.
template <bool BF16>
__global__ __launch_bounds__(NT) void im2col_kernel(const Im2colLayer* layers, int n, int64_t tiles) {
    const int64_t item = xcd_remap(blockIdx.x, gridDim.x);
    if (item >= tiles) return;
    const Im2colLayer L = layers[find_layer(layers, n, item, &Im2colLayer::tile_begin)];
    const int64_t t = item - L.tile_begin;
    const int64_t tr = t / L.tiles_c;
    const int tc = (int)(t % L.tiles_c);
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    const int col = T * tc + tx;
    if (col >= L.cols) return;
    const int core = L.cols - L.ones;
    const bool one = col >= core;
    const int taps = L.kh * L.kw;
    const int ci = one ? 0 : col / taps, rem = one ? 0 : col % taps;
    const int di = (rem / L.kw) * L.dh - L.ph, dj = (rem % L.kw) * L.dw - L.pw;
    int64_t r = T * tr + ty;
    const int64_t per = (int64_t)L.oh * L.ow;
    int64_t ni = r / per;
    int q = (int)(r % per);
    int y = q / L.ow, x = q % L.ow;
    using E = typename std::conditional<BF16, uint16_t, float>::type;
    const E* X = static_cast<const E*>(L.x);
    E* A = static_cast<E*>(L.a);
    E unit;
    if constexpr (BF16) unit = (uint16_t)0x3f80u;
    else unit = 1.0f;
#pragma unroll 4
    for (int s = 0; s < T / 4; ++s, r += 4) {
        if (r >= L.rows) break;
        E v = unit;
        if (!one) {
            const int yy = y * L.sh + di, xx = x * L.sw + dj;
            v = (E)0;
            if (yy >= 0 && yy < L.h && xx >= 0 && xx < L.w) v = X[((ni * L.c + ci) * L.h + yy) * L.w + xx];
        }
        A[r * L.cols + col] = v;
        x += 4;
        while (x >= L.ow) {
            x -= L.ow;
            if (++y == L.oh) {
                y = 0;
                ++ni;
            }
        }
    }
}

template <bool BF16>
__device__ __forceinline__ float load_val(const void* p, int64_t i) {
    if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    else return static_cast<const float*>(p)[i];
}
template <bool BF16>
__device__ __forceinline__ void store_val(void* p, int64_t i, float v) {
    if constexpr (BF16) static_cast<uint16_t*>(p)[i] = f32_to_bf16_rne(v);
    else static_cast<float*>(p)[i] = v;
}

// hw > 1: tile (b, channels 64 tc.., positions 64 tp..) transposed through
// LDS, read along positions and written along channels.  hw == 1: tile
// (samples 64 tp.., channels 64 tc..), a scaled copy along channels.
template <bool BF16>
__global__ __launch_bounds__(NT) void grad_rows_kernel(const GradRowsLayer* layers, int n, int64_t tiles,
                                                       float scale) {
    __shared__ float S[T][T + 1];
    const int64_t item = xcd_remap(blockIdx.x, gridDim.x);
    if (item >= tiles) return;
    const GradRowsLayer L = layers[find_layer(layers, n, item, &GradRowsLayer::tile_begin)];
    const int64_t t = item - L.tile_begin;
    const int lx = threadIdx.x & 63, ly = threadIdx.x >> 6;
    if (L.hw == 1) {
        const int64_t b0 = (t / L.tiles_c) * T;
        const int64_t c0 = (t % L.tiles_c) * T;
        const int64_t ci = c0 + lx;
        if (ci >= L.c) return;
        for (int s = 0; s < T / 4; ++s) {
            const int64_t b = b0 + ly + 4 * s;
            if (b < L.batch) store_val<BF16>(L.g, b * L.c + ci, scale * load_val<BF16>(L.gy, b * L.c + ci));
        }
        return;
    }
    const int64_t per = (int64_t)L.tiles_c * L.tiles_p;
    const int64_t b = t / per;
    const int64_t c0 = ((t % per) / L.tiles_p) * T;
    const int64_t p0 = ((t % per) % L.tiles_p) * T;
    for (int s = 0; s < T / 4; ++s) {   // rows = channels, lanes = positions
        const int64_t ci = c0 + ly + 4 * s, p = p0 + lx;
        S[ly + 4 * s][lx] = (ci < L.c && p < L.hw) ? load_val<BF16>(L.gy, (b * L.c + ci) * L.hw + p) : 0.0f;
    }
    __syncthreads();
    for (int s = 0; s < T / 4; ++s) {   // rows = positions, lanes = channels
        const int64_t p = p0 + ly + 4 * s, ci = c0 + lx;
        if (p < L.hw && ci < L.c) store_val<BF16>(L.g, (b * L.hw + p) * L.c + ci, scale * S[lx][ly + 4 * s]);
    }
}

// kGradMatChunk consecutive elements of mat[l] per workgroup.
__global__ __launch_bounds__(NT) void grad_matrix_kernel(const GradMatLayer* layers, int n, int64_t chunks,
                                                         int pack) {
    const int64_t item = xcd_remap(blockIdx.x, gridDim.x);
    if (item >= chunks) return;
    const GradMatLayer L = layers[find_layer(layers, n, item, &GradMatLayer::chunk_begin)];
    const int64_t total = L.d_out * L.cols;
    const int64_t e0 = (item - L.chunk_begin) * kGradMatChunk;
    for (int s = 0; s < kGradMatChunk / NT; ++s) {
        const int64_t e = e0 + threadIdx.x + (int64_t)s * NT;
        if (e >= total) break;
        const int64_t r = e / L.cols, k = e % L.cols;
        float* src = k < L.d_in ? L.w + r * L.d_in + k : L.b + r;
        if (pack) L.mat[e] = *src;
        else *src = L.mat[e];
    }
}

}  // namespace

hipError_t launch_im2col(const Im2colLayer* layers, int n, int64_t tiles, bool bf16, hipStream_t stream) {
    if (tiles <= 0) return hipSuccess;
    if (bf16) hipLaunchKernelGGL(im2col_kernel<true>, dim3((unsigned)tiles), dim3(NT), 0, stream, layers, n, tiles);
    else hipLaunchKernelGGL(im2col_kernel<false>, dim3((unsigned)tiles), dim3(NT), 0, stream, layers, n, tiles);
    return hipGetLastError();
}

hipError_t launch_grad_rows(const GradRowsLayer* layers, int n, int64_t tiles, bool bf16, float scale,
                            hipStream_t stream) {
    if (tiles <= 0) return hipSuccess;
    if (bf16)
        hipLaunchKernelGGL(grad_rows_kernel<true>, dim3((unsigned)tiles), dim3(NT), 0, stream, layers, n, tiles, scale);
    else
        hipLaunchKernelGGL(grad_rows_kernel<false>, dim3((unsigned)tiles), dim3(NT), 0, stream, layers, n, tiles, scale);
    return hipGetLastError();
}

hipError_t launch_grad_matrix(const GradMatLayer* layers, int n, int64_t chunks, bool pack, hipStream_t stream) {
    if (chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(grad_matrix_kernel, dim3((unsigned)chunks), dim3(NT), 0, stream, layers, n, chunks, pack ? 1 : 0);
    return hipGetLastError();
}

}  // namespace kfac
