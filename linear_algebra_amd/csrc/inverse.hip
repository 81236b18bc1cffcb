// Damped SPD inverse Z = (X + gamma I)^-1 for a batch of matrices of mixed
// size, in float64 on the matrix cores (v_mfma_f64_16x16x4f64).
//
// Each matrix is padded with the identity to D = nb * 64 and processed in
// 64 x 64 blocks in a float64 workspace W (row-major D x D):
//
//   prepare   W = sym(X) + gamma I (upper blocks), and the Cholesky of the
//             first diagonal block;
//   potrf     for k = 0 .. nb-2 (right-looking, upper: Y = U^T U)
//               trsm  U_kj = U_kk^-T W_kj           (j > k)
//               syrk  W_ij -= U_ki^T U_kj           (k < i <= j); the
//                     workgroup that updates block (k+1, k+1) then factors it
//                     (Cholesky in LDS) and inverts its triangle;
//   trtri     V = U^-1 by recursive doubling over groups of blocks: for
//             sibling groups G1, G2 (G1 before G2)
//               V_12 = -V_11 . (U_12 . V_22)
//             two launches per level, log2(nb) levels; the inner product is
//             parked in the unused lower triangle of W;
//   lauum     Z = V V^T (upper blocks), written as float32 to both triangles.
//
// Diagonal blocks of V are the inverses of the diagonal blocks of U, kept in
// a separate array (dinv).  Matrices are grouped in buckets of equal nb,
// largest first; every launch covers every matrix that has work at that
// step, so independent inverses of different layers run side by side.
#include "device_common.h"
#include "internal.h"

namespace kfac {
namespace {

constexpr int B = kInvNB;      // block edge
constexpr int LD = B + 1;      // LDS row stride in doubles (conflict-free columns)
constexpr int NT = kInvThreads;
constexpr int BB = B * B;

// Which matrix and which of its tiles a workgroup owns.
__device__ __forceinline__ bool locate(const InvLaunch& L, int kind, int64_t tile, int& mat, int64_t& local) {
    for (int b = 0; b < L.nbuckets; ++b) {
        const InvBucket bk = L.buckets[b];
        const int64_t per = inv_tiles(kind, bk.nb, L.step);
        const int64_t cnt = per * bk.count;
        if (tile < cnt) {
            mat = bk.first + (int)(tile / per);
            local = tile % per;
            return true;
        }
        tile -= cnt;
    }
    return false;
}

// S[m][k] <- G block (64 x 64, leading dimension ld); `trans` stores G^T.
// Global reads run along G's rows (coalesced) in both cases.
__device__ __forceinline__ void load_block(double* S, const double* G, int64_t ld, bool trans) {
    for (int e = threadIdx.x; e < BB; e += NT) {
        const int r = e >> 6, c = e & 63;
        const double v = G[(int64_t)r * ld + c];
        if (trans) S[c * LD + r] = v; else S[r * LD + c] = v;
    }
}

// acc[m][n] += (neg ? -1 : 1) * sum_k As[m][k] * Bs[n][k] over one 64-deep block.
// Wave w owns the 32 x 32 quadrant (w/2, w%2) as 2 x 2 MFMA blocks of 16 x 16.
__device__ __forceinline__ void mma_block(doublex4 (&acc)[2][2], const double* As, const double* Bs, bool neg) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int li = lane & 15, lk = lane >> 4;
    const double* a0p = As + (wr * 32 + li) * LD + lk;
    const double* a1p = a0p + 16 * LD;
    const double* b0p = Bs + (wc * 32 + li) * LD + lk;
    const double* b1p = b0p + 16 * LD;
#pragma unroll 4
    for (int k0 = 0; k0 < B; k0 += 4) {
        double a0 = a0p[k0], a1 = a1p[k0];
        const double b0 = b0p[k0], b1 = b1p[k0];
        if (neg) { a0 = -a0; a1 = -a1; }
        acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
    }
}

// Output layout of a 16 x 16 f64 MFMA block (checked on gfx950): lane l holds
// column l % 16 and rows l/16 + 4*r for its four registers r.  (The f32
// 16 x 16 blocks use rows 4*(l/16) + r instead.)
template <typename F>
__device__ __forceinline__ void for_acc(F&& f) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wr = wave >> 1, wc = wave & 1;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                f(a, b, r, wr * 32 + a * 16 + (lane >> 4) + 4 * r, wc * 32 + b * 16 + (lane & 15));
}

__device__ __forceinline__ void acc_zero(doublex4 (&acc)[2][2]) {
    for_acc([&](int a, int b, int r, int, int) { acc[a][b][r] = 0.0; });
}
__device__ __forceinline__ void acc_load(doublex4 (&acc)[2][2], const double* G, int64_t ld) {
    for_acc([&](int a, int b, int r, int row, int col) { acc[a][b][r] = G[(int64_t)row * ld + col]; });
}
__device__ __forceinline__ void acc_store(const doublex4 (&acc)[2][2], double* G, int64_t ld) {
    for_acc([&](int a, int b, int r, int row, int col) { G[(int64_t)row * ld + col] = acc[a][b][r]; });
}
__device__ __forceinline__ void acc_to_lds(const doublex4 (&acc)[2][2], double* S) {
    for_acc([&](int a, int b, int r, int row, int col) { S[row * LD + col] = acc[a][b][r]; });
}

// In-place Cholesky P = U^T U of a 64 x 64 block in LDS (upper triangle
// read and written).  Returns 0, or the 1-based column of the first pivot
// that is not positive or not finite.  Caller synchronises before the call.
__device__ int panel_cholesky(double* P) {
    int failed = 0;
    for (int c = 0; c < B; ++c) {
        const double piv = P[c * LD + c];
        if (failed == 0 && (!(piv > 0.0) || !isfinite(piv))) failed = c + 1;
        const double r = sqrt(piv);
        __syncthreads();  // every thread has read the pivot
        for (int j = c + (int)threadIdx.x; j < B; j += NT) P[c * LD + j] = (j == c) ? r : P[c * LD + j] / r;
        __syncthreads();
        const int m = B - 1 - c;
        for (int e = threadIdx.x; e < m * m; e += NT) {
            const int i = c + 1 + e / m, j = c + 1 + e % m;
            if (j >= i) P[i * LD + j] -= P[c * LD + i] * P[c * LD + j];
        }
        __syncthreads();
    }
    return failed;
}

// V = U^-1 for the upper-triangular 64 x 64 block U in LDS (V upper, zero
// below the diagonal).  Column j is solved backwards by the four threads
// 4j .. 4j+3, which split each inner product and combine it with shuffles;
// all four write the same value, so each reads back only its own writes.
__device__ void triangle_inverse(const double* U, double* V) {
    const int j = threadIdx.x >> 2, p = threadIdx.x & 3;
    for (int i = j + 1 + p; i < B; i += 4) V[i * LD + j] = 0.0;
    V[j * LD + j] = 1.0 / U[j * LD + j];
    for (int i = j - 1; i >= 0; --i) {
        double s = 0.0;
        for (int t = i + 1 + p; t <= j; t += 4) s += U[i * LD + t] * V[t * LD + j];
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        V[i * LD + j] = -s / U[i * LD + i];
    }
    __syncthreads();
}

// Factor the diagonal block held in P (LDS), invert its triangle into Q,
// store U (zero below the diagonal) into W's block and U^-1 into dinv.
// Returns the 1-based failing column inside the block, or 0.
__device__ int factor_diagonal_block(double* P, double* Q, double* Wkk, int64_t D, double* dinv_k) {
    __syncthreads();
    const int f = panel_cholesky(P);
    triangle_inverse(P, Q);
    for (int e = threadIdx.x; e < BB; e += NT) {
        const int r = e >> 6, c = e & 63;
        Wkk[(int64_t)r * D + c] = (c >= r) ? P[r * LD + c] : 0.0;
        dinv_k[e] = Q[r * LD + c];
    }
    return f;
}

__device__ __forceinline__ void record_info(const InvMat& M, int k, int f, bool first_panel) {
    if (threadIdx.x != 0) return;
    if (first_panel) {
        *M.info = f ? f : 0;
    } else if (f && *M.info == 0) {
        *M.info = k * B + f;
    }
}

// -------------------------------------------------------------- kernels --

__global__ __launch_bounds__(NT) void inv_prepare_kernel(InvLaunch L, int64_t tiles) {
    __shared__ double P[B * LD];
    __shared__ double Q[B * LD];
    int mi;
    int64_t local;
    if (!locate(L, kInvPrepare, blockIdx.x, mi, local)) return;
    const InvMat M = L.mats[mi];
    int bi, bj;
    upper_decode(local, M.nb, bi, bj);
    const int64_t D = (int64_t)M.nb * B, d = M.d;
    const bool first = (bi == 0 && bj == 0);
    for (int e = threadIdx.x; e < BB; e += NT) {
        const int r = e >> 6, c = e & 63;
        const int64_t i = (int64_t)bi * B + r, j = (int64_t)bj * B + c;
        double v;
        if (i < d && j < d) {
            v = (j >= i) ? (double)M.x[i * d + j] : 0.0;
            if (i == j) v += L.gamma;
        } else {
            v = (i == j) ? 1.0 : 0.0;  // identity padding
        }
        if (first) P[r * LD + c] = v; else M.w[i * D + j] = v;
    }
    if (first) {
        const int f = factor_diagonal_block(P, Q, M.w, D, M.dinv);
        record_info(M, 0, f, true);
    }
}

__global__ __launch_bounds__(NT) void inv_trsm_kernel(InvLaunch L, int64_t tiles) {
    __shared__ double As[B * LD];
    __shared__ double Bs[B * LD];
    int mi;
    int64_t local;
    if (!locate(L, kInvTrsm, blockIdx.x, mi, local)) return;
    const InvMat M = L.mats[mi];
    const int k = L.step;
    const int J = k + 1 + (int)local;
    const int64_t D = (int64_t)M.nb * B;
    double* Wkj = M.w + (int64_t)k * B * D + (int64_t)J * B;
    load_block(As, M.dinv + (int64_t)k * BB, B, true);   // A[r][t] = Uinv_kk[t][r]
    load_block(Bs, Wkj, D, true);                        // B[c][t] = W_kj[t][c]
    __syncthreads();
    doublex4 acc[2][2];
    acc_zero(acc);
    mma_block(acc, As, Bs, false);
    acc_store(acc, Wkj, D);
}

__global__ __launch_bounds__(NT) void inv_syrk_kernel(InvLaunch L, int64_t tiles) {
    __shared__ double As[B * LD];
    __shared__ double Bs[B * LD];
    int mi;
    int64_t local;
    if (!locate(L, kInvSyrk, blockIdx.x, mi, local)) return;
    const InvMat M = L.mats[mi];
    const int k = L.step;
    const int T = M.nb - k - 1;
    int a, b;
    upper_decode(local, T, a, b);
    const int I = k + 1 + a, J = k + 1 + b;
    const int64_t D = (int64_t)M.nb * B;
    double* Wij = M.w + (int64_t)I * B * D + (int64_t)J * B;
    const double* rowk = M.w + (int64_t)k * B * D;
    doublex4 acc[2][2];
    acc_load(acc, Wij, D);
    load_block(As, rowk + (int64_t)I * B, D, true);      // A[r][t] = U_ki[t][r]
    if (I != J) load_block(Bs, rowk + (int64_t)J * B, D, true);
    __syncthreads();
    mma_block(acc, As, (I == J) ? As : Bs, true);
    if (I == k + 1 && J == k + 1) {
        __syncthreads();
        acc_to_lds(acc, As);
        const int f = factor_diagonal_block(As, Bs, Wij, D, M.dinv + (int64_t)I * BB);
        record_info(M, I, f, false);
    } else {
        acc_store(acc, Wij, D);
    }
}

// Tile of level `lvl` of the doubling: group m joins G1 = [m*2h, m*2h + h)
// and G2 = [m*2h + h, min(m*2h + 2h, nb)); the tile is block (I, J),
// I in G1, J in G2.
__device__ __forceinline__ void trtri_decode(int64_t local, int nb, int lvl, int& I, int& J, int& g1_end) {
    const int h = 1 << (lvl - 1), g = 2 * h;
    const int full = nb / g;
    const int64_t hh = (int64_t)h * h;
    int m, bi, bj;
    if (local / hh < full) {
        m = (int)(local / hh);
        const int r = (int)(local % hh);
        bi = r / h;
        bj = r % h;
    } else {
        m = full;
        const int r = (int)(local - (int64_t)full * hh);
        const int w2 = nb % g - h;
        bi = r / w2;
        bj = r % w2;
    }
    I = m * g + bi;
    J = m * g + h + bj;
    g1_end = m * g + h;
}

// T_IJ = sum_{t in G2, t <= J} U_It V_tJ, parked in W's lower block (J, I).
__global__ __launch_bounds__(NT) void inv_trtri_a_kernel(InvLaunch L, int64_t tiles) {
    __shared__ double As[B * LD];
    __shared__ double Bs[B * LD];
    int mi;
    int64_t local;
    if (!locate(L, kInvTrtri, blockIdx.x, mi, local)) return;
    const InvMat M = L.mats[mi];
    int I, J, g1_end;
    trtri_decode(local, M.nb, L.step, I, J, g1_end);
    const int64_t D = (int64_t)M.nb * B;
    doublex4 acc[2][2];
    acc_zero(acc);
    for (int t = g1_end; t <= J; ++t) {
        __syncthreads();
        load_block(As, M.w + (int64_t)I * B * D + (int64_t)t * B, D, false);          // U_It
        if (t == J) load_block(Bs, M.dinv + (int64_t)J * BB, B, true);                // V_JJ
        else load_block(Bs, M.w + (int64_t)t * B * D + (int64_t)J * B, D, true);     // V_tJ
        __syncthreads();
        mma_block(acc, As, Bs, false);
    }
    acc_store(acc, M.w + (int64_t)J * B * D + (int64_t)I * B, D);
}

// V_IJ = - sum_{t in G1, t >= I} V_It T_tJ, written over U_IJ.
__global__ __launch_bounds__(NT) void inv_trtri_b_kernel(InvLaunch L, int64_t tiles) {
    __shared__ double As[B * LD];
    __shared__ double Bs[B * LD];
    int mi;
    int64_t local;
    if (!locate(L, kInvTrtri, blockIdx.x, mi, local)) return;
    const InvMat M = L.mats[mi];
    int I, J, g1_end;
    trtri_decode(local, M.nb, L.step, I, J, g1_end);
    const int64_t D = (int64_t)M.nb * B;
    doublex4 acc[2][2];
    acc_zero(acc);
    for (int t = I; t < g1_end; ++t) {
        __syncthreads();
        if (t == I) load_block(As, M.dinv + (int64_t)I * BB, B, false);               // V_II
        else load_block(As, M.w + (int64_t)I * B * D + (int64_t)t * B, D, false);     // V_It
        load_block(Bs, M.w + (int64_t)J * B * D + (int64_t)t * B, D, true);           // T_tJ (parked at (J, t))
        __syncthreads();
        mma_block(acc, As, Bs, true);
    }
    acc_store(acc, M.w + (int64_t)I * B * D + (int64_t)J * B, D);
}

// Z_IJ = sum_{t >= J} V_It V_Jt^T for I <= J; float32 out, both triangles.
__global__ __launch_bounds__(NT) void inv_lauum_kernel(InvLaunch L, int64_t tiles) {
    __shared__ double As[B * LD];
    __shared__ double Bs[B * LD];
    int mi;
    int64_t local;
    if (!locate(L, kInvLauum, blockIdx.x, mi, local)) return;
    const InvMat M = L.mats[mi];
    int I, J;
    upper_decode(local, M.nb, I, J);
    const int64_t D = (int64_t)M.nb * B, d = M.d;
    doublex4 acc[2][2];
    acc_zero(acc);
    for (int t = J; t < M.nb; ++t) {
        __syncthreads();
        if (t == I) load_block(As, M.dinv + (int64_t)I * BB, B, false);
        else load_block(As, M.w + (int64_t)I * B * D + (int64_t)t * B, D, false);
        if (I != J) {
            if (t == J) load_block(Bs, M.dinv + (int64_t)J * BB, B, false);
            else load_block(Bs, M.w + (int64_t)J * B * D + (int64_t)t * B, D, false);
        }
        __syncthreads();
        mma_block(acc, As, (I == J) ? As : Bs, false);
    }
    __syncthreads();
    acc_to_lds(acc, As);
    __syncthreads();
    const int64_t r0 = (int64_t)I * B, c0 = (int64_t)J * B;
    for (int e = threadIdx.x; e < BB; e += NT) {
        const int r = e >> 6, c = e & 63;
        const int64_t i = r0 + r, j = c0 + c;
        if (i < d && j < d) {
            const double v = (I != J || c >= r) ? As[r * LD + c] : As[c * LD + r];
            M.z[i * d + j] = (float)v;
        }
    }
    if (I != J) {
        for (int e = threadIdx.x; e < BB; e += NT) {
            const int c = e >> 6, r = e & 63;     // destination row c0+c, column r0+r
            const int64_t i = c0 + c, j = r0 + r;
            if (i < d && j < d) M.z[i * d + j] = (float)As[r * LD + c];
        }
    }
}

template <typename K>
hipError_t launch(K kernel, const InvLaunch& L, int64_t tiles, hipStream_t s) {
    if (tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(kernel, dim3((unsigned)tiles), dim3(NT), 0, s, L, tiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_inv_prepare(const InvLaunch& L, int64_t t, hipStream_t s) { return launch(inv_prepare_kernel, L, t, s); }
hipError_t launch_inv_trsm(const InvLaunch& L, int64_t t, hipStream_t s) { return launch(inv_trsm_kernel, L, t, s); }
hipError_t launch_inv_syrk(const InvLaunch& L, int64_t t, hipStream_t s) { return launch(inv_syrk_kernel, L, t, s); }
hipError_t launch_inv_trtri_a(const InvLaunch& L, int64_t t, hipStream_t s) { return launch(inv_trtri_a_kernel, L, t, s); }
hipError_t launch_inv_trtri_b(const InvLaunch& L, int64_t t, hipStream_t s) { return launch(inv_trtri_b_kernel, L, t, s); }
hipError_t launch_inv_lauum(const InvLaunch& L, int64_t t, hipStream_t s) { return launch(inv_lauum_kernel, L, t, s); }

}  // namespace kfac
