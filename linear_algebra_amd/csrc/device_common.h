// Device-side helpers shared by the kernels of the K-FAC library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kfac {

// A pointer into global memory as such, so that its accesses are global
// (not flat) instructions: they count only against the vector-memory wait
// counter, and a wait for LDS or scalar loads does not also wait for them.
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T* as_global(T* p) {
    return (__attribute__((address_space(1))) T*)p;
}


typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef double doublex4 __attribute__((ext_vector_type(4)));

// Work items are numbered so that neighbours share input data.  The hardware
// hands consecutive workgroups to the 8 XCDs in turn, and each XCD has its
// own L2; this remap gives every XCD one contiguous range of items instead,
// so neighbouring items run under the same L2.  It is a bijection on
// [0, count).
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t count) {
    const int64_t x = b & 7, local = b >> 3;
    const int64_t q = count >> 3, r = count & 7;
    if (count < 8) return b;
    return x * q + (x < r ? x : r) + local;
}

// For launches whose items differ in cost (long and short products), a
// contiguous range per XCD leaves some XCDs with far more work than others.
// Here the XCDs take runs of C consecutive items in turn (XCD x gets runs x,
// x + 8, ...), which keeps neighbours together and balances the load.  The
// grid must be a multiple of 8 C; it is a bijection on [0, gridDim.x).
template <int C>
__device__ __forceinline__ int64_t xcd_runs(int64_t b) {
    const int64_t x = b & 7, local = b >> 3;
    return ((local / C) * 8 + x) * C + local % C;
}

// Row-major enumeration of the upper triangle (i <= j) of a T x T grid:
// row i holds T - i entries.  t in [0, T(T+1)/2).
__device__ __forceinline__ void upper_decode(int64_t t, int64_t T, int& i, int& j) {
    // closed form from the quadratic, then fix-ups for rounding
    const double a = 2.0 * (double)T + 1.0;
    int64_t r = (int64_t)((a - sqrt(a * a - 8.0 * (double)t)) * 0.5);
    if (r < 0) r = 0;
    if (r > T - 1) r = T - 1;
    while (r > 0 && r * T - r * (r - 1) / 2 > t) --r;
    while (r + 1 < T && (r + 1) * T - (r + 1) * r / 2 <= t) ++r;
    i = (int)r;
    j = (int)(r + (t - (r * T - r * (r - 1) / 2)));
}

// Column-by-column enumeration of an upper triangle: t = j(j+1)/2 + i with
// 0 <= i <= j, so column j holds j + 1 entries.
__device__ __forceinline__ void column_decode(int64_t t, int& i, int& j) {
    int64_t r = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
    if (r < 0) r = 0;
    while (r > 0 && r * (r + 1) / 2 > t) --r;
    while ((r + 1) * (r + 2) / 2 <= t) ++r;
    j = (int)r;
    i = (int)(t - r * (r + 1) / 2);
}

// Banded enumeration of the upper triangle (i <= j) of a T x T grid: bands
// of `band` rows, column by column within a band (the band's first `band`
// columns form a triangle), so that band^2 consecutive entries form about
// a band x band block.  t in [0, T(T+1)/2); a band occupies the same range
// of t as its rows do in row-major order.
__device__ __forceinline__ void upper_band_decode(int64_t t, int64_t T, int band, int& i, int& j) {
    int ir, jr;
    upper_decode(t, T, ir, jr);   // the row-major position gives the band
    const int64_t i0 = (int64_t)(ir / band) * band;
    const int64_t r = min<int64_t>(band, T - i0);
    const int64_t u = t - (i0 * T - i0 * (i0 - 1) / 2);
    const int64_t tri = r * (r + 1) / 2;
    if (u < tri) {
        int a, c;
        column_decode(u, a, c);
        i = (int)(i0 + a);
        j = (int)(i0 + c);
    } else {
        const int64_t v = u - tri;
        i = (int)(i0 + v % r);
        j = (int)(i0 + r + v / r);
    }
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

}  // namespace kfac
