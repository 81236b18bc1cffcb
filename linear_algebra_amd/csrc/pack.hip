// Triangular pack / unpack between per-layer d x d float32 matrices and one
// fused float32 buffer holding their upper triangles (incl. the diagonal),
// row by row, layers back to back.  Both directions are bit-exact copies.
//
// Layer offsets.  The host uploads only (pointer, order) per factor.  One
// wavefront turns them into the layer table: the packed offset of a layer is
// the exclusive prefix sum of d (d + 1) / 2 over the layers before it, and
// its first unpack tile the prefix sum of T (T + 1) / 2, T = ceil(d / 64);
// both are computed 64 layers at a time by a scan across the lanes, carried
// from one group of 64 to the next.
//
// Pack.  The fused buffer is cut into 16-byte units that start on a 16-byte
// boundary (the at most three elements before the first boundary and after
// the last are copied one by one).  A lane takes one unit per step: the row
// of its first element comes from the closed form of the row start,
// i d - i (i - 1) / 2; when the four elements lie in one row they are read
// with one 16-byte load (rows start at any 4-byte boundary), otherwise
// element by element.  Every lane issues the loads of its four units before
// any store.  A workgroup covers 2048 consecutive packed elements and finds
// the layers it touches once; only a workgroup that straddles a layer
// boundary looks a layer up per unit.
//
// Unpack.  One workgroup per 64 x 64 tile of the upper block triangle of a
// matrix; each thread moves a 4 x 4 block of it: four 16-byte row loads
// from the fused buffer, four 16-byte row stores in place, and four more of
// the block's columns (transposed in registers) into the mirrored tile.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace kfac {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

// 16-byte global accesses at 4-byte aligned addresses (the rows of a d x d
// matrix start on a 16-byte boundary only when d is a multiple of 4).
__device__ __forceinline__ f4 load4(const float* p) {
    f4 v;
    __builtin_memcpy(&v, p, sizeof(v));
    return v;
}
__device__ __forceinline__ void store4(float* p, f4 v) { __builtin_memcpy(p, &v, sizeof(v)); }

constexpr int PT = kPackThreads;
constexpr int PU = kPackUnits;
constexpr int UT = kUnpackTile;

__device__ __forceinline__ int64_t row_start(int64_t i, int64_t d) { return i * d - i * (i - 1) / 2; }

// Row of the upper triangle of a d x d matrix that holds local packed index
// q: the quadratic's root in float64 (exact operands for d <= 16384), then
// integer checks settle it.
__device__ __forceinline__ int64_t row_of(int64_t q, int64_t d) {
    const double a = 2.0 * (double)d + 1.0;
    int64_t i = (int64_t)((a - sqrt(a * a - 8.0 * (double)q)) * 0.5);
    i = i < 0 ? 0 : (i > d - 1 ? d - 1 : i);
    while (i > 0 && row_start(i, d) > q) --i;
    while (i + 1 < d && row_start(i + 1, d) <= q) ++i;
    return i;
}

// Largest layer l in [lo, hi] with key(l) <= e (keys ascending).
template <bool kByTile>
__device__ __forceinline__ int find_layer(const PackLayer* L, int lo, int hi, int64_t e) {
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        const int64_t b = kByTile ? L[mid].tile_begin : L[mid].off;
        if (b <= e) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// One packed element, located from scratch (layer, row, column).
__device__ float packed_element(const PackLayer* L, int n, int64_t e) {
    const PackLayer& P = L[find_layer<false>(L, 0, n - 1, e)];
    const int64_t q = e - P.off, i = row_of(q, P.d);
    return P.m[i * P.d + i + (q - row_start(i, P.d))];
}

// The four packed elements from local index q of one layer (q + 3 inside
// the layer): one 16-byte load when they share a row, else one by one,
// stepping from the end of a row to the diagonal of the next.
__device__ __forceinline__ f4 unit_in_layer(const float* m, int64_t d, int64_t q) {
    const int64_t i = row_of(q, d);
    const int64_t j = i + (q - row_start(i, d));
    if (j + 3 < d) return load4(m + i * d + j);
    f4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        int64_t r = i, c = j + k;
        while (c >= d) {            // past the end of row r: row r + 1 starts at its diagonal
            c = c - d + r + 1;
            ++r;
        }
        v[k] = m[r * d + c];
    }
    return v;
}

__global__ __launch_bounds__(64) void pack_table_kernel(const PackSrc* __restrict__ src, int n,
                                                        PackLayer* __restrict__ out) {
    const int lane = threadIdx.x;
    int64_t carry_e = 0, carry_t = 0;
    for (int base = 0; base < n; base += 64) {
        const int l = base + lane;
        float* m = nullptr;
        int64_t d = 0;
        if (l < n) {
            m = src[l].m;
            d = src[l].d;
        }
        const int64_t T = (d + UT - 1) / UT;
        const int64_t own_e = d * (d + 1) / 2, own_t = T * (T + 1) / 2;
        int64_t e = own_e, t = own_t;   // inclusive scan across the wavefront
#pragma unroll
        for (int s = 1; s < 64; s <<= 1) {
            const int64_t pe = __shfl_up(e, s, 64), pt = __shfl_up(t, s, 64);
            if (lane >= s) {
                e += pe;
                t += pt;
            }
        }
        if (l < n) out[l] = PackLayer{m, d, carry_e + e - own_e, carry_t + t - own_t, T};
        carry_e += __shfl(e, 63, 64);
        carry_t += __shfl(t, 63, 64);
    }
}

// Units u cover packed elements [head + 4u, head + 4u + 4), 16-byte aligned
// in memory; `head` elements come before the first unit and at most three
// after the last.
__global__ __launch_bounds__(PT) void pack_kernel(const PackLayer* __restrict__ layers, int n,
                                                  float* __restrict__ packed, int64_t total, int64_t head,
                                                  int64_t units) {
    if (blockIdx.x == 0 && threadIdx.x < 8) {
        const int64_t e = threadIdx.x < 4 ? threadIdx.x : head + 4 * units + (threadIdx.x - 4);
        const bool mine = threadIdx.x < 4 ? e < head : e < total;
        if (mine) packed[e] = packed_element(layers, n, e);
    }
    const int64_t u0 = (int64_t)blockIdx.x * (PT * PU);
    if (u0 >= units) return;
    const int64_t u_end = u0 + PT * PU < units ? u0 + PT * PU : units;
    const int lf = find_layer<false>(layers, 0, n - 1, head + 4 * u0);
    const int ll = find_layer<false>(layers, lf, n - 1, head + 4 * (u_end - 1) + 3);
    f4 v[PU];
    if (lf == ll) {
        // the whole workgroup inside one layer (its fields are uniform)
        const float* m = layers[lf].m;
        const int64_t d = layers[lf].d, off = layers[lf].off;
#pragma unroll
        for (int s = 0; s < PU; ++s) {
            const int64_t u = u0 + threadIdx.x + PT * s;
            if (u < units) v[s] = unit_in_layer(m, d, head + 4 * u - off);
        }
    } else {
#pragma unroll
        for (int s = 0; s < PU; ++s) {
            const int64_t u = u0 + threadIdx.x + PT * s;
            if (u < units) {
                const int64_t e = head + 4 * u;
                const PackLayer& P = layers[find_layer<false>(layers, lf, ll, e)];
                if (e + 3 < P.off + P.d * (P.d + 1) / 2) {
                    v[s] = unit_in_layer(P.m, P.d, e - P.off);
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) v[s][k] = packed_element(layers, n, e + k);
                }
            }
        }
    }
#pragma unroll
    for (int s = 0; s < PU; ++s) {
        const int64_t u = u0 + threadIdx.x + PT * s;
        if (u < units) store4(packed + head + 4 * u, v[s]);
    }
}

// Each thread of a tile owns one 4 x 4 sub-block: it reads the block's four
// rows from the fused buffer (16-byte loads), writes them in place, and
// writes the block's columns as rows of the mirrored tile (the transpose
// happens in registers).  A wave takes an 8 x 8 square of sub-blocks, so
// that each of its loads and stores, in place or mirrored, covers 128
// contiguous bytes of 8 rows.  On a diagonal tile only the sub-blocks on or
// above the diagonal work; one on the diagonal fills its lower half from its
// upper half.
__global__ __launch_bounds__(256) void unpack_kernel(const PackLayer* __restrict__ layers, int n,
                                                     const float* __restrict__ packed, int64_t tiles) {
    // a contiguous range of tiles per XCD: the tiles that share a cache line
    // at the ends of their row segments (neighbours in a tile row, and in a
    // tile column of the mirror) then write it through the same L2
    const int64_t tile = xcd_remap(blockIdx.x, gridDim.x);
    if (tile >= tiles) return;
    const PackLayer& P = layers[find_layer<true>(layers, 0, n - 1, tile)];
    int ti, tj;
    upper_decode(tile - P.tile_begin, P.tiles_1d, ti, tj);
    const int64_t d = P.d;
    float* const m = P.m;
    const float* const src = packed + P.off;
    const int w = threadIdx.x >> 6, t = threadIdx.x & 63;
    const int a = 8 * (w & 1) + (t & 7), b = 8 * (w >> 1) + (t >> 3);   // sub-block row and column
    if (ti == tj && b < a) return;   // below the diagonal of a diagonal tile: done by its mirror
    const int64_t R = (int64_t)ti * UT + 4 * a, C = (int64_t)tj * UT + 4 * b;   // block origin
    if (R >= d) return;              // only on a diagonal tile at the matrix's edge (C >= R)
    const bool cfull = C + 3 < d;    // all four columns inside the matrix
    f4 v[4];
    if (ti != tj || a != b) {
        // the whole block lies above the diagonal (C >= R + 4)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = R + i;
            v[i] = f4{0.0f, 0.0f, 0.0f, 0.0f};
            if (r < d) {
                const float* p = src + row_start(r, d) + (C - r);
                if (cfull) {
                    v[i] = load4(p);
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) v[i][k] = C + k < d ? p[k] : 0.0f;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (R + i >= d) continue;
            float* q = m + (R + i) * d + C;
            if (cfull) {
                store4(q, v[i]);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (C + k < d) q[k] = v[i][k];
            }
        }
        // mirror: row C + k holds column k of the block, at columns R .. R + 3
        const bool rfull = R + 3 < d;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (C + k >= d) continue;
            float* q = m + (C + k) * d + R;
            const f4 w = {v[0][k], v[1][k], v[2][k], v[3][k]};
            if (rfull) {
                store4(q, w);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (R + i < d) q[i] = w[i];
            }
        }
    } else {
        // a block on the diagonal (R == C): entries (i, k >= i) from the
        // fused buffer, the rest their mirrors
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v[i][k] = 0.0f;
                if (k >= i && R + k < d) v[i][k] = src[row_start(R + i, d) + (k - i)];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < i; ++k) v[i][k] = v[k][i];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (R + i >= d) continue;
            float* q = m + (R + i) * d + C;
            if (cfull) {
                store4(q, v[i]);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (C + k < d) q[k] = v[i][k];
            }
        }
    }
}

// Plain device copy, one 16-byte unit per lane, 256 lanes per workgroup:
// of the shapes measured (one to sixteen units per lane, 256 to 1024 lanes
// per workgroup, persistent grid-stride loops, non-temporal stores) the
// fastest on MI355X.
__global__ __launch_bounds__(PT) void stream_copy_kernel(const f4* __restrict__ src, f4* __restrict__ dst,
                                                         int64_t units) {
    const int64_t u = (int64_t)blockIdx.x * PT + threadIdx.x;
    if (u < units) dst[u] = src[u];
}

}  // namespace

hipError_t launch_pack_table(const PackSrc* src, int n, PackLayer* out, hipStream_t stream) {
    hipLaunchKernelGGL(pack_table_kernel, dim3(1), dim3(64), 0, stream, src, n, out);
    return hipGetLastError();
}

hipError_t launch_pack(const PackLayer* layers, int n, float* packed, int64_t total, hipStream_t stream) {
    if (total <= 0) return hipSuccess;
    const int64_t mis = (int64_t)((reinterpret_cast<uintptr_t>(packed) & 15) >> 2);   // packed is 4-byte aligned
    const int64_t head = std::min<int64_t>(total, (4 - mis) & 3);
    const int64_t units = (total - head) / 4;
    const int64_t blocks = std::max<int64_t>(1, ceil_div(units, (int64_t)PT * PU));
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(PT), 0, stream, layers, n, packed, total, head, units);
    return hipGetLastError();
}

hipError_t launch_unpack(const PackLayer* layers, int n, const float* packed, int64_t tiles, hipStream_t stream) {
    if (tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, layers, n, packed, tiles);
    return hipGetLastError();
}

hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
    const int64_t units = (int64_t)(bytes / 16);
    if (units == 0) return hipSuccess;
    const int64_t blocks = ceil_div(units, (int64_t)PT);
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(PT), 0, stream, static_cast<const f4*>(src),
                       static_cast<f4*>(dst), units);
    return hipGetLastError();
}

}  // namespace kfac
