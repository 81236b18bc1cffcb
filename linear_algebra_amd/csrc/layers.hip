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

template <typename E>
using Vec4 = E __attribute__((ext_vector_type(4)));

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
template <bool BF16>
__device__ __forceinline__ float to_f32(typename std::conditional<BF16, uint16_t, float>::type v) {
    if constexpr (BF16) return bf16_to_f32(v);
    else return v;
}
template <bool BF16>
__device__ __forceinline__ typename std::conditional<BF16, uint16_t, float>::type from_f32(float v) {
    if constexpr (BF16) return f32_to_bf16_rne(v);
    else return v;
}

// Both layer transposes stage a 64 x 64 tile in LDS as S[column][row]
// (row stride 65, so that reading a column of S is free of bank conflicts).
// The four-element forms give thread t the rows 4 (t % 16) .. + 3 of the
// columns t / 16 + 16 k when gathering, and the columns 4 (t % 16) .. + 3 of
// the rows t / 16 + 16 k when writing: a wave then moves 4 x 64 consecutive
// elements per access.

// One 64 x 64 tile of a[l].  Gather: lanes = rows (sample, output y, output
// x), so a wave reads along output x, which is contiguous in x[l] for stride
// 1; the column (channel and kernel tap) of each gather is uniform over the
// wave.  Write: lanes = columns, so a wave writes along one row of a[l].
template <bool BF16>
__global__ __launch_bounds__(NT) void im2col_kernel(const Im2colLayer* layers, int n, int64_t tiles) {
    using E = typename std::conditional<BF16, uint16_t, float>::type;
    using V = Vec4<E>;
    __shared__ E S[T][T + 1];
    const int64_t item = xcd_remap(blockIdx.x, gridDim.x);
    if (item >= tiles) return;
    const Im2colLayer L = layers[find_layer(layers, n, item, &Im2colLayer::tile_begin)];
    const int64_t t = item - L.tile_begin;
    const int64_t r0 = (t / L.tiles_c) * T;
    const int c0 = (int)(t % L.tiles_c) * T;
    const int lx = threadIdx.x & 63;
    const int ly = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int q4 = threadIdx.x & 15, g16 = threadIdx.x >> 4;
    const E* X = static_cast<const E*>(L.x);
    E* A = static_cast<E*>(L.a);
    E unit;
    if constexpr (BF16) unit = (uint16_t)0x3f80u;
    else unit = 1.0f;
    const int64_t plane = L.h * L.w;
    const int core = L.cols - L.ones;

    // Every gather loads, from element 0 of x[l] when its source is padding
    // or past the last row, and selects afterwards: with no branch around
    // the loads, all of a thread's gathers are in flight at once.
    if (L.vec & kVecIn) {
        // 1 x 1 kernel, stride 1, no padding, h w % 4 == 0: rows r .. r + 3
        // (r % 4 == 0) are positions q .. q + 3 of one sample
        const int64_t r = r0 + 4 * q4;
        const bool rok = r < L.rows;
        const int64_t ni = r / plane;
        const int64_t base = ni * L.c * plane + (r - ni * plane);
        V v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int col = c0 + g16 + 16 * k;
            const bool ok = rok && col < core;
            v[k] = *reinterpret_cast<const V*>(X + (ok ? base + col * plane : 0));
            if (!ok) v[k] = col < core ? (V)(E)0 : (V)unit;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int cl = g16 + 16 * k;
            S[cl][4 * q4 + 0] = v[k].x;
            S[cl][4 * q4 + 1] = v[k].y;
            S[cl][4 * q4 + 2] = v[k].z;
            S[cl][4 * q4 + 3] = v[k].w;
        }
    } else {
        const int64_t r = r0 + lx;
        const bool rok = r < L.rows;
        const int64_t per = (int64_t)L.oh * L.ow;
        const int64_t ni = rok ? r / per : 0;
        const int q = (int)(r - ni * per);
        const int y0 = (q / L.ow) * L.sh - L.ph, x0 = (q % L.ow) * L.sw - L.pw;
        const E* Xn = X + ni * L.c * plane;   // element 0 of sample ni (of sample 0 past the last row)
        // lane l decodes column c0 + l (channel, tap offsets) once; gather s
        // takes the decode of its column from lane ly + 4 s
        const int taps = L.kh * L.kw;
        const int mycol = c0 + lx;
        const int myci = mycol / taps, myrem = mycol - myci * taps;
        const int mydi = (myrem / L.kw) * L.dh, mydj = (myrem % L.kw) * L.dw;
        E v[T / 4];
#pragma unroll
        for (int s = 0; s < T / 4; ++s) {
            const int src = ly + 4 * s;
            const int col = c0 + src;
            const int ci = __builtin_amdgcn_readlane(myci, src);
            const int yy = y0 + __builtin_amdgcn_readlane(mydi, src);
            const int xx = x0 + __builtin_amdgcn_readlane(mydj, src);
            const bool ok = rok && col < core && (unsigned)yy < (unsigned)L.h && (unsigned)xx < (unsigned)L.w;
            // c h w < 2^31: the offset inside one sample fits 32 bits
            v[s] = Xn[ok ? ci * (int)plane + yy * (int)L.w + xx : 0];
            if (!ok) v[s] = col < core ? (E)0 : unit;
        }
#pragma unroll
        for (int s = 0; s < T / 4; ++s) S[ly + 4 * s][lx] = v[s];
    }
    __syncthreads();
    if (L.vec & kVecOut) {
        // cols % 4 == 0: a column group is inside a[l] or wholly past its end
        const int col = c0 + 4 * q4;
        if (col >= L.cols) return;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int rl = g16 + 16 * k;
            const int64_t rr = r0 + rl;
            if (rr < L.rows) {
                const V v = {S[4 * q4][rl], S[4 * q4 + 1][rl], S[4 * q4 + 2][rl], S[4 * q4 + 3][rl]};
                *reinterpret_cast<V*>(A + rr * L.cols + col) = v;
            }
        }
        return;
    }
    const int col = c0 + lx;
    if (col >= L.cols) return;
#pragma unroll 4
    for (int s = 0; s < T / 4; ++s) {
        const int64_t rr = r0 + ly + 4 * s;
        if (rr < L.rows) A[rr * L.cols + col] = S[lx][ly + 4 * s];
    }
}

// hw > 1: tile (b, channels 64 tc.., positions 64 tp..) transposed through
// LDS, read along positions and written along channels.  hw == 1: tile
// (samples 64 tp.., channels 64 tc..), a scaled copy along channels.
template <bool BF16>
__global__ __launch_bounds__(NT) void grad_rows_kernel(const GradRowsLayer* layers, int n, int64_t tiles,
                                                       float scale) {
    using E = typename std::conditional<BF16, uint16_t, float>::type;
    using V = Vec4<E>;
    __shared__ float S[T][T + 1];
    const int64_t item = xcd_remap(blockIdx.x, gridDim.x);
    if (item >= tiles) return;
    const GradRowsLayer L = layers[find_layer(layers, n, item, &GradRowsLayer::tile_begin)];
    const int64_t t = item - L.tile_begin;
    const int lx = threadIdx.x & 63, ly = threadIdx.x >> 6;
    const int q4 = threadIdx.x & 15, g16 = threadIdx.x >> 4;
    if (L.hw == 1) {   // all loads first (from element 0 past the edges), then the stores
        const int64_t b0 = (t / L.tiles_c) * T;
        const int64_t c0 = (t % L.tiles_c) * T;
        const int64_t ci = c0 + lx;
        float v[T / 4];
#pragma unroll
        for (int s = 0; s < T / 4; ++s) {
            const int64_t b = b0 + ly + 4 * s;
            v[s] = load_val<BF16>(L.gy, (b < L.batch && ci < L.c) ? b * L.c + ci : 0);
        }
        if (ci >= L.c) return;
#pragma unroll
        for (int s = 0; s < T / 4; ++s) {
            const int64_t b = b0 + ly + 4 * s;
            if (b < L.batch) store_val<BF16>(L.g, b * L.c + ci, scale * v[s]);
        }
        return;
    }
    const int64_t per = (int64_t)L.tiles_c * L.tiles_p;
    const int64_t b = t / per;
    const int64_t c0 = ((t % per) / L.tiles_p) * T;
    const int64_t p0 = ((t % per) % L.tiles_p) * T;
    const E* GY = static_cast<const E*>(L.gy);
    E* G = static_cast<E*>(L.g);
    // loads from element 0 of gy[l] outside the tile's range, selects after
    if (L.vec & kVecIn) {   // hw % 4 == 0: a position group is in range or wholly past hw
        const int64_t p = p0 + 4 * q4;
        V v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t ci = c0 + g16 + 16 * k;
            const bool ok = ci < L.c && p < L.hw;
            v[k] = *reinterpret_cast<const V*>(GY + (ok ? (b * L.c + ci) * L.hw + p : 0));
            if (!ok) v[k] = (V)(E)0;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int cl = g16 + 16 * k;
            S[cl][4 * q4 + 0] = to_f32<BF16>(v[k].x);
            S[cl][4 * q4 + 1] = to_f32<BF16>(v[k].y);
            S[cl][4 * q4 + 2] = to_f32<BF16>(v[k].z);
            S[cl][4 * q4 + 3] = to_f32<BF16>(v[k].w);
        }
    } else {
        float v[T / 4];
#pragma unroll
        for (int s = 0; s < T / 4; ++s) {   // rows = channels, lanes = positions
            const int64_t ci = c0 + ly + 4 * s, p = p0 + lx;
            const bool ok = ci < L.c && p < L.hw;
            v[s] = load_val<BF16>(GY, ok ? (b * L.c + ci) * L.hw + p : 0);
            if (!ok) v[s] = 0.0f;
        }
#pragma unroll
        for (int s = 0; s < T / 4; ++s) S[ly + 4 * s][lx] = v[s];
    }
    __syncthreads();
    if (L.vec & kVecOut) {   // c % 4 == 0
        const int64_t ci = c0 + 4 * q4;
        if (ci >= L.c) return;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int pl = g16 + 16 * k;
            const int64_t p = p0 + pl;
            if (p < L.hw) {
                const V v = {from_f32<BF16>(scale * S[4 * q4][pl]), from_f32<BF16>(scale * S[4 * q4 + 1][pl]),
                             from_f32<BF16>(scale * S[4 * q4 + 2][pl]), from_f32<BF16>(scale * S[4 * q4 + 3][pl])};
                *reinterpret_cast<V*>(G + (b * L.hw + p) * L.c + ci) = v;
            }
        }
        return;
    }
    for (int s = 0; s < T / 4; ++s) {   // rows = positions, lanes = channels
        const int64_t p = p0 + ly + 4 * s, ci = c0 + lx;
        if (p < L.hw && ci < L.c) store_val<BF16>(G, (b * L.hw + p) * L.c + ci, scale * S[lx][ly + 4 * s]);
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
    // every element read before any is written (a read after a write to a
    // buffer that might alias would wait for it); reads past the end take
    // element 0 of the source
    constexpr int PER = kGradMatChunk / NT;
    float* src[PER];
    float v[PER];
#pragma unroll
    for (int s = 0; s < PER; ++s) {
        const int64_t e = e0 + threadIdx.x + (int64_t)s * NT;
        const int64_t ec = e < total ? e : 0;
        const int64_t r = ec / L.cols, k = ec % L.cols;
        src[s] = k < L.d_in ? L.w + r * L.d_in + k : L.b + r;
        v[s] = pack ? *as_global(src[s]) : as_global(L.mat)[ec];
    }
#pragma unroll
    for (int s = 0; s < PER; ++s) {
        const int64_t e = e0 + threadIdx.x + (int64_t)s * NT;
        if (e >= total) break;
        if (pack) as_global(L.mat)[e] = v[s];
        else *as_global(src[s]) = v[s];
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
