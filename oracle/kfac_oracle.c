/*
 * kfac_oracle.c -- TEST INFRASTRUCTURE ONLY.  A plain, slow, fp64 CPU
 * reference for the parts of the K-FAC hot path that numpy cannot express as
 * a single library call: the triangular pack / unpack index map and the
 * Cholesky-based damped inverse.  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg load this file's library.  It shares no
 * code, header or constant with the GPU library.
 *
 * Sources (page: "Accelerating Distributed K-FAC with Smart Parallelism of
 * Computing and Communication Tasks"):
 *   - damped inverse (X + gamma I)^-1: the paragraph on Tikhonov
 *     regularisation before inverting (the update rule with damping
 *     parameter gamma), and the paragraph on the inverse being computed
 *     through a Cholesky decomposition (cuSolver via CuPy);
 *   - upper-triangle packing, d(d+1)/2 elements including the diagonal:
 *     the paragraph on sending only the upper triangles of the symmetric
 *     inverses, and the tensor-fusion paragraph on the number of
 *     communicated elements of a symmetric factor.
 *
 * Conventions (readings where the page is silent):
 *   - matrices are row-major; "upper" means entries (i, j) with j >= i;
 *   - the packed order is row by row through the upper triangle, layers
 *     concatenated in call order, no padding;
 *   - a failed factorisation reports info = k (1-based), the order of the
 *     first leading minor whose pivot is not positive or not finite, as the
 *     LAPACK xPOTRF routines do.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- pack -- */

int64_t oracle_packed_size(int n, const int64_t* d)
{
    int64_t s = 0;
    for (int l = 0; l < n; ++l) s += d[l] * (d[l] + 1) / 2;
    return s;
}

/* packed[off_l + (row i of the upper triangle) + (j - i)] = M_l[i][j], j >= i.
 * Values are moved as 32-bit patterns: the map is a pure copy. */
void oracle_pack(int n, const uint32_t* const* m, const int64_t* d, uint32_t* packed)
{
    int64_t p = 0;
    for (int l = 0; l < n; ++l) {
        const int64_t dl = d[l];
        for (int64_t i = 0; i < dl; ++i)
            for (int64_t j = i; j < dl; ++j) packed[p++] = m[l][i * dl + j];
    }
}

/* Inverse map: every packed element goes back to (i, j) and to (j, i). */
void oracle_unpack(int n, const uint32_t* packed, const int64_t* d, uint32_t* const* m)
{
    int64_t p = 0;
    for (int l = 0; l < n; ++l) {
        const int64_t dl = d[l];
        for (int64_t i = 0; i < dl; ++i)
            for (int64_t j = i; j < dl; ++j) {
                const uint32_t v = packed[p++];
                m[l][i * dl + j] = v;
                m[l][j * dl + i] = v;
            }
    }
}

/* ------------------------------------------------------------ Cholesky -- */

/* In-place Cholesky Y = U^T U of the symmetric matrix whose upper triangle
 * is stored in y (row-major, d x d).  On return the upper triangle holds U;
 * the strict lower triangle is not touched.  Outer-product (right-looking)
 * column order: take the pivot, scale its row, subtract the rank-one update
 * from the trailing upper triangle.  Returns 0, or the 1-based order of the
 * first pivot that is not positive or not finite. */
int64_t oracle_cholesky_upper(double* y, int64_t d)
{
    for (int64_t k = 0; k < d; ++k) {
        const double p = y[k * d + k];
        if (!(p > 0.0) || !isfinite(p)) return k + 1;
        const double r = sqrt(p);
        double* uk = y + k * d;
        uk[k] = r;
        for (int64_t j = k + 1; j < d; ++j) uk[j] = uk[j] / r;
#pragma omp parallel for schedule(static) if (d - k > 192)
        for (int64_t i = k + 1; i < d; ++i) {
            const double uki = uk[i];
            double* yi = y + i * d;
            for (int64_t j = i; j < d; ++j) yi[j] -= uki * uk[j];
        }
    }
    return 0;
}

/* Column c of Y^-1 from the factor U: solve U^T w = e_c (forward, w_i = 0
 * for i < c), then U z = w (backward).  z has d entries. */
static void solve_column(const double* u, int64_t d, int64_t c, double* w, double* z)
{
    for (int64_t i = 0; i < d; ++i) w[i] = 0.0;
    w[c] = 1.0;
    for (int64_t k = c; k < d; ++k) {
        const double* uk = u + k * d;
        w[k] = w[k] / uk[k];
        const double wk = w[k];
        for (int64_t i = k + 1; i < d; ++i) w[i] -= uk[i] * wk;
    }
    for (int64_t i = d - 1; i >= 0; --i) {
        const double* ui = u + i * d;
        double s = w[i];
        for (int64_t k = i + 1; k < d; ++k) s -= ui[k] * z[k];
        z[i] = s / ui[i];
    }
}

/* Y = (upper triangle of x, read as a symmetric matrix) + gamma I, in the
 * upper triangle of y. */
static void damp(const double* x, int64_t d, double gamma, double* y)
{
    for (int64_t i = 0; i < d; ++i) {
        for (int64_t j = 0; j < i; ++j) y[i * d + j] = 0.0;
        for (int64_t j = i; j < d; ++j) y[i * d + j] = x[i * d + j];
        y[i * d + i] += gamma;
    }
}

/* Selected columns of (X + gamma I)^-1.  out[q * d + r] = Z[r][cols[q]].
 * Returns info (0 on success; out is then filled). */
int64_t oracle_damped_inverse_columns(const double* x, int64_t d, double gamma,
                                      const int64_t* cols, int64_t ncols, double* out)
{
    double* y = (double*)malloc((size_t)(d * d) * sizeof(double));
    if (!y) return -1;
    damp(x, d, gamma, y);
    const int64_t info = oracle_cholesky_upper(y, d);
    if (info == 0) {
#pragma omp parallel
        {
            double* w = (double*)malloc((size_t)d * sizeof(double));
#pragma omp for schedule(dynamic, 1)
            for (int64_t q = 0; q < ncols; ++q) solve_column(y, d, cols[q], w, out + q * d);
            free(w);
        }
    }
    free(y);
    return info;
}

/* Full (X + gamma I)^-1, row-major: z[r * d + c] = Z[r][c].  Returns info. */
int64_t oracle_damped_inverse(const double* x, int64_t d, double gamma, double* z)
{
    double* y = (double*)malloc((size_t)(d * d) * sizeof(double));
    if (!y) return -1;
    damp(x, d, gamma, y);
    const int64_t info = oracle_cholesky_upper(y, d);
    if (info == 0) {
#pragma omp parallel
        {
            double* w = (double*)malloc((size_t)d * sizeof(double));
            double* col = (double*)malloc((size_t)d * sizeof(double));
#pragma omp for schedule(dynamic, 1)
            for (int64_t c = 0; c < d; ++c) {
                solve_column(y, d, c, w, col);
                for (int64_t r = 0; r < d; ++r) z[r * d + c] = col[r];
            }
            free(col);
            free(w);
        }
    }
    free(y);
    return info;
}
