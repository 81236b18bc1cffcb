// Damped SPD inverse Z = (X + gamma I)^-1 for a batch of matrices of mixed
// size, in float64 on the matrix cores (v_mfma_f64_16x16x4f64).
//
// Each matrix is padded with the identity to D = nb * 64 and processed in
// 64 x 64 blocks in a float64 workspace W (row-major D x D):
//
//   prepare   W = sym(X) + gamma I (upper blocks), identity in the padding;
//   potrf     right-looking, upper (Y = U^T U), one launch per step k with
//             a look-ahead of one step:
//               row k     W_kj -= sum_p U_pk^T U_pj  (j >= k, p in [plo, k));
//                         then every row-k workgroup factors the diagonal
//                         block and inverts its triangle (16-row strips, see
//                         factor_diagonal) and solves one block of the row:
//                         U_kj = U_kk^-T W_kj           (j > k)
//               trailing  W_ij -= sum_p U_pi^T U_pj  (k < i <= j, p in
//                         [plo, k)), in the same launch, beside the row-k
//                         workgroups; where the trailing matrix is large the
//                         host runs it only every second or third step, so
//                         that one read and write of a block takes two or
//                         three panels (plo is the first panel not applied);
//   V = U^-1  formed one of two ways, chosen by the host from the trailing
//             work per step:
//             fused     beside potrf: at step k the blocks of column k-1
//                         above the diagonal get partial sums
//                         sum_m V_im U_m,k-1 over chunks of two panels, and
//                         column k-2 is finished as
//                         V_ic = -(sum of its partials) V_cc; V_ic is kept
//                         in the lower block (c, i), two extra launches
//                         finish the last columns;
//             trtri     after potrf, by recursive doubling over groups of
//                         blocks, from the leaves up: for sibling groups G1,
//                         G2 (G1 before G2)  V_12 = -V_11 . (U_12 . V_22),
//                         two launches per level, ceil(log2(nb)) levels; the
//                         groups are runs of 2^l blocks, or a balanced binary
//                         tree when nb is just above a power of two; the
//                         inner product is parked in the lower triangle of W;
//   border    for an order d = 64m + 1 (d > 64), only the leading 64m x 64m
//             part goes through the steps above; its last row and column are
//             attached afterwards as one more (bordered) Cholesky step, by two
//             matrix-vector launches, and the last product adds v v^T for
//             the border column v of V;
//   V V^T     Z = V V^T: V^T rounded to float32 (vt32), then the float32
//             GEMM of the factor stage (products as six bf16 products of
//             exact splits), upper tiles with K from max(row, column), both
//             triangles written (see inv_vt32_kernel for why float32
//             suffices here).
//
// Diagonal blocks of V are the inverses of the diagonal blocks of U, kept in
// a separate array (dinv).  Matrices are grouped in buckets of equal nb,
// largest first; every launch covers every matrix that has work at that
// step, so independent inverses of different layers run side by side.
//
// Block products stage their operands in LDS in halves of 32 k-columns,
// double buffered: the load units copy the next half straight into LDS
// while the matrix cores work on the current one.
#include <float.h>

#include "device_common.h"
#include "internal.h"

namespace kfac {
namespace {

constexpr int B = kInvNB;      // block edge
constexpr int LD = B + 1;      // LDS row stride in doubles (conflict-free columns)
constexpr int NT = kInvThreads;
constexpr int BB = B * B;
constexpr int PER = BB / NT;   // block elements per thread (16)
constexpr int kRun = 16;       // items per XCD run in launches of uneven items (trtri)

// Which matrix and which of its tiles a workgroup owns.
__device__ __forceinline__ bool locate(const InvLaunch& L, int kind, int64_t tile, int& mat, int64_t& local) {
    for (int b = 0; b < L.nbuckets; ++b) {
        const InvBucket bk = L.buckets[b];
        const int64_t per = inv_tiles(kind, bk.nb, L.step, kind == kInvPanel ? L.rowq : 1);
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

// A 64 x 64 block in global memory; `trans` stages it transposed in LDS.
struct Blk {
    const double* p;
    int64_t ld;
    bool trans;
};

// Thread t handles elements e = t + s*NT: row e/64, column e%64, so each
// wave reads whole 512-byte rows.
__device__ __forceinline__ void fetch(double (&v)[PER], const Blk& b) {
    const int r0 = threadIdx.x >> 6, c = threadIdx.x & 63;
#pragma unroll
    for (int s = 0; s < PER; ++s) v[s] = as_global(b.p)[(int64_t)(r0 + 4 * s) * b.ld + c];
}
__device__ __forceinline__ void put(double* S, const double (&v)[PER], bool trans) {
    const int r0 = threadIdx.x >> 6, c = threadIdx.x & 63;
    if (trans) {
#pragma unroll
        for (int s = 0; s < PER; ++s) S[c * LD + r0 + 4 * s] = v[s];
    } else {
#pragma unroll
        for (int s = 0; s < PER; ++s) S[(r0 + 4 * s) * LD + c] = v[s];
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
#pragma unroll
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

// Products of many blocks stage their operands in halves of 32 k-columns,
// double buffered, one barrier per half.  The load units copy each half
// from global memory straight into LDS (16 bytes per lane,
// global_load_lds_dwordx4), so the data never passes through registers:
// the loads of the next half are issued right after the barrier that frees
// its buffer and land while the matrix cores work on the current one.  Four
// staged halves (A and B, two buffers each) take 64 KB, so two workgroups
// still share a CU.
constexpr int KH = 32;            // k-columns per half
constexpr int HD = B * KH;        // doubles per staged half (unpadded)

// The staging area: two LDS arrays, which hold the A and B halves of
// buffer 0 and of buffer 1 (the first is a padded 64 x 64 block, which the
// epilogues also use).  They are separate arrays, not one, so that the
// compiler can tell the copies into one buffer from the reads of the other
// and does not wait for the copies first.
constexpr int SLOT = B * LD;
static_assert(SLOT >= 2 * HD, "the A and B halves of a buffer fit in one array");
struct Stage {
    double* s0;
    double* s1;
};

// Layouts of a staged piece of K k-columns (K = 32: a half, K = 16: a
// quarter), as [m][k] (for an untransposed block m is its row and k its
// column, for a transposed one the reverse):
//   untransposed: row m holds its K / 2 pairs of k-values, pair k/2 at
//     position (k/2) xor (m & 7), so the 16 rows an operand fragment reads
//     at one k fall on 8 bank groups instead of one;
//   transposed: [k][m], m contiguous, as the block's rows lie in memory.
template <int K>
__device__ __forceinline__ int staged_at(bool trans, int m, int k) {
    return trans ? k * B + m : m * K + ((((k >> 1) ^ (m & 7)) << 1) | (k & 1));
}

// Issues the copy of piece q (k-columns [K q, K q + K)) of block b into S
// (B K doubles).  Wave w, instruction s fills pairs 64 (n w + s) + lane of
// the layout; each lane fetches the pair that belongs there, so every row
// segment of the block is read by consecutive lanes.
template <int K>
__device__ __forceinline__ void stage_piece(double* S, const Blk& b, int q) {
    constexpr int n = B * K / (2 * NT);   // copy instructions per wave
    constexpr int rowpairs = K / 2;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int s = 0; s < n; ++s) {
        const int first = (n * w + s) * 64;
        const int p = first + lane;
        const double* src;
        if (!b.trans) {
            const int m = p / rowpairs, c = (p % rowpairs) ^ (m & 7);
            src = b.p + (int64_t)m * b.ld + K * q + 2 * c;
        } else {
            const int k = p >> 5, mc = p & 31;
            src = b.p + (int64_t)(K * q + k) * b.ld + 2 * mc;
        }
        __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                         (void __attribute__((address_space(3)))*)(S + 2 * first), 16, 0, 0);
    }
}

// The k-values k and k + 1 (k even) of row m of a staged piece.  Untransposed
// they are one 16-byte pair; transposed they sit in consecutive k-rows.
template <int K>
__device__ __forceinline__ double2 frag_pair(const double* S, bool trans, int m, int k) {
    if (!trans) return *reinterpret_cast<const double2*>(S + staged_at<K>(false, m, k));
    return make_double2(S[staged_at<K>(true, m, k)], S[staged_at<K>(true, m, k + 1)]);
}

// acc[m][n] += (neg ? -1 : 1) * sum_k A[m][k] B[n][k] over one staged piece;
// the wave layout of mma_block.  The sum does not depend on which k-values
// each MFMA takes, so every lane group reads a pair of them at once: in
// steps of 8 k-values, lane group g (lanes 16 g .. 16 g + 15) takes k0 + 2 g
// in the first product and k0 + 2 g + 1 in the second.  An untransposed
// operand is then one 16-byte read per row, whole swizzled pairs, which
// meet no bank conflict (8-byte reads of one half of each pair can reach
// only half of the banks).
template <int K>
__device__ __forceinline__ void mma_staged(doublex4 (&acc)[2][2], const double* A, bool ta, const double* Bm, bool tb,
                                           bool neg) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int li = lane & 15, lk = lane >> 4;
    const int ma = wr * 32 + li, nb = wc * 32 + li;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 8) {
        const int k = k0 + 2 * lk;
        double2 a0 = frag_pair<K>(A, ta, ma, k), a1 = frag_pair<K>(A, ta, ma + 16, k);
        const double2 b0 = frag_pair<K>(Bm, tb, nb, k), b1 = frag_pair<K>(Bm, tb, nb + 16, k);
        if (neg) {
            a0.x = -a0.x; a0.y = -a0.y;
            a1.x = -a1.x; a1.y = -a1.y;
        }
        acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0.x, b0.x, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0.x, b1.x, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1.x, b0.x, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1.x, b1.x, acc[1][1], 0, 0, 0);
        acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0.y, b0.y, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0.y, b1.y, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1.y, b0.y, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1.y, b1.y, acc[1][1], 0, 0, 0);
    }
}

// A barrier that waits only for the workgroup's LDS accesses: unlike
// __syncthreads() it lets global loads stay in flight (the block a caller
// loaded into registers before a product, and the product's first copies,
// then travel together).  The memory clobber keeps the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt and expcnt left at their maximum
    asm volatile("s_barrier" ::: "memory");
}

// acc += (neg ? -1 : 1) sum_{t in [t0, t1)} A_t B_t^T, A_t and B_t the
// 64 x 64 blocks srcA(t), srcB(t) (staged as [m][k]); `same` reuses A for B.
// Each block is staged in 64 / K pieces of K k-columns; even pieces go
// through buffer 0, odd ones through buffer 1 (each buffer holds the A and
// B pieces, 2 B K doubles, at the start of its array).  For each piece: wait
// for its copies, barrier (its data is visible, and the other buffer, read
// by the piece before, is free), issue the copies of the next piece into
// the other buffer, multiply.  Ends with a barrier, so the staging area may
// be reused at once.
template <int K = KH, typename FA, typename FB>
__device__ __forceinline__ void block_gemm(doublex4 (&acc)[2][2], const Stage& S, int t0, int t1, FA srcA, FB srcB,
                                           bool neg, bool same) {
    constexpr int P = B / K;   // pieces per block, even
    constexpr int PD = B * K;  // doubles per staged piece
    static_assert(P % 2 == 0, "pieces alternate between the buffers within a block");
    if (t0 >= t1) return;
    // offsets, not a choice of pointers, so that each stays visibly inside
    // its array
    double* const A0 = S.s0;
    double* const B0 = S.s0 + (same ? 0 : PD);
    double* const A1 = S.s1;
    double* const B1 = S.s1 + (same ? 0 : PD);
    lds_barrier();   // earlier users of the staging area are done
    stage_piece<K>(A0, srcA(t0), 0);
    if (!same) stage_piece<K>(B0, srcB(t0), 0);
    const int pieces = P * (t1 - t0);
    for (int j = 0; j < pieces; j += 2) {
        const int t = t0 + j / P, q = j % P;   // pieces q (buffer 0) and q + 1 (buffer 1) of block t
        const bool ta = srcA(t).trans, tb = same ? ta : srcB(t).trans;
        __builtin_amdgcn_s_waitcnt(0);   // the copies of piece j (the only loads in flight)
        __syncthreads();
        stage_piece<K>(A1, srcA(t), q + 1);
        if (!same) stage_piece<K>(B1, srcB(t), q + 1);
        mma_staged<K>(acc, A0, ta, B0, tb, neg);
        __builtin_amdgcn_s_waitcnt(0);   // the copies of piece j + 1
        __syncthreads();
        if (j + 2 < pieces) {
            const int tn = t0 + (j + 2) / P, qn = (j + 2) % P;
            stage_piece<K>(A0, srcA(tn), qn);
            if (!same) stage_piece<K>(B0, srcB(tn), qn);
        }
        mma_staged<K>(acc, A1, ta, B1, tb, neg);
    }
    __syncthreads();
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
    for_acc([&](int a, int b, int r, int row, int col) { acc[a][b][r] = as_global(G)[(int64_t)row * ld + col]; });
}
__device__ __forceinline__ void acc_store(const doublex4 (&acc)[2][2], double* G, int64_t ld) {
    for_acc([&](int a, int b, int r, int row, int col) { as_global(G)[(int64_t)row * ld + col] = acc[a][b][r]; });
}
__device__ __forceinline__ void acc_to_lds(const doublex4 (&acc)[2][2], double* S) {
    for_acc([&](int a, int b, int r, int row, int col) { S[row * LD + col] = acc[a][b][r]; });
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), lane);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// 1/sqrt(x) to double precision: the hardware estimate (relative error
// about 5e-8) refined by one third-order step, y <- y + y r (1/2 + 3/8 r)
// with r = 1 - x y^2 (the series of (1 - r)^(-1/2)), which cubes the error;
// four dependent operations on the pivot chain.
__device__ __forceinline__ double rsqrt_refined(double x) {
    const double y = __builtin_amdgcn_rsq(x);
    const double r = fma(-x * y, y, 1.0);
    return fma(y * r, fma(0.375, r, 0.5), y);
}

constexpr int SB = 16;          // strip height and leaf block edge
constexpr int NS = B / SB;      // strips per diagonal block

// LDS scratch of factor_diagonal: the pivot row being broadcast, one
// failure slot per strip.
struct PanelScratch {
    alignas(16) double row[B];   // the current pivot row of the strip being factored
    int fail[NS];
};

// acc += (neg ? -1 : 1) A B over K = 16 for 16 x 16 blocks in LDS (row
// stride LD): A[i][k] = X[xr + i][xc + k], or X[xr + k][xc + i] when `at`;
// B[k][j] = Y[yr + k][yc + j], or Y[yr + j][yc + k] when `bt`.  Lane l feeds A[l % 16][4c + l / 16] and
// B[4c + l / 16][l % 16] to k-chunk c of v_mfma_f64_16x16x4f64.
__device__ __forceinline__ void mm16(doublex4& acc, const double* X, int xr, int xc, bool at, const double* Y,
                                     int yr, int yc, bool neg, bool bt = false) {
    const int l = threadIdx.x & 63, li = l & 15, lk = l >> 4;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
        const int k = 4 * kc + lk;
        double a = at ? X[(xr + k) * LD + xc + li] : X[(xr + li) * LD + xc + k];
        const double b = bt ? Y[(yr + li) * LD + yc + k] : Y[(yr + k) * LD + yc + li];
        if (neg) a = -a;
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc, 0, 0, 0);
    }
}
// 16 x 16 block <-> accumulator (lane l: column l % 16, rows l / 16 + 4r).
__device__ __forceinline__ void load16(doublex4& acc, const double* X, int r0, int c0) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = X[(r0 + (l >> 4) + 4 * r) * LD + c0 + (l & 15)];
}
__device__ __forceinline__ void store16(const doublex4& acc, double* X, int r0, int c0) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int r = 0; r < 4; ++r) X[(r0 + (l >> 4) + 4 * r) * LD + c0 + (l & 15)] = acc[r];
}
__device__ __forceinline__ doublex4 zero4() {
    doublex4 z;
    z[0] = z[1] = z[2] = z[3] = 0.0;
    return z;
}

// Cholesky of strip s (rows SB*s .. SB*s + 15 of the diagonal block, already
// updated by the strips above it).  Lane j holds column (SB*s + j) mod 64 in
// u[0..15], so the strip's own diagonal block sits in lanes 0..15; the
// wrapped lanes (columns left of the strip) carry values nobody reads.
// Pivot c takes the diagonal entry from lane c, scales row c by its inverse
// square root and subtracts the rank-one update from the rows below.  Row
// c + 1 gets its update first, through a cross-lane read, so that pivot
// c + 1's square-root chain runs beside the other rows' updates, which read
// row c back from LDS (same address in every lane, all reads in flight at
// once).
//
// The same rows of U give the inverse of the strip's diagonal block,
// V = U_ss^-1, by forward elimination on V U = I: lane i keeps row i % 16 of
// V in x[0..15] (starting as that row of the identity); after pivot c,
// x[c] *= 1 / U_cc and x[t] -= x[c] U_ct for t > c.  This rides on the
// pivot loop's reads of row c and fills the issue slots the square-root
// chain leaves idle.  Returns the 1-based column of the first pivot that is
// not positive or not finite, or 0.
__device__ __forceinline__ int strip_factor(double (&u)[SB], double (&x)[SB], PanelScratch& S, int s, int j) {
    int failed = 0;
    double piv = readlane_f64(u[0], 0);
    double yc = rsqrt_refined(piv);
#pragma unroll
    for (int c = 0; c < SB; ++c) x[c] = ((j & (SB - 1)) == c) ? 1.0 : 0.0;
#pragma unroll
    for (int c = 0; c < SB; ++c) {
        failed = (failed == 0 && !(piv > 0.0 && piv <= DBL_MAX)) ? SB * s + c + 1 : failed;
        u[c] *= yc;   // lane c holds the pivot itself: U_cc = piv / sqrt(piv)
        x[c] *= yc;
        if (c + 1 < SB) {
            if (c + 2 < SB) S.row[j] = u[c];
            const double r1 = readlane_f64(u[c], c + 1);   // U_c,c+1
            u[c + 1] = fma(-r1, u[c], u[c + 1]);
            x[c + 1] = fma(-r1, x[c], x[c + 1]);
            // row c in pairs, every read in flight at once
            double2 rp[SB / 2];
#pragma unroll
            for (int p = (c + 2) / 2; p < SB / 2; ++p) rp[p] = reinterpret_cast<const double2*>(S.row)[p];
            const double pn = readlane_f64(u[c + 1], c + 1);
            const double yn = rsqrt_refined(pn);
#pragma unroll
            for (int t = c + 2; t < SB; ++t) {
                const double rt = (t & 1) ? rp[t / 2].y : rp[t / 2].x;   // U_ct
                u[t] = fma(-rt, u[c], u[t]);
                x[t] = fma(-rt, x[c], x[t]);
            }
            piv = pn;
            yc = yn;
        }
        // keep each step's reads within the step: hoisted, they hold too
        // many registers
        __builtin_amdgcn_sched_barrier(0);
    }
    return failed;
}

// Block (i, c) of V = U^-1 from the blocks of V to its left and the
// diagonal block V_cc (V U = I):  V_ic = -(sum_{i <= m < c} V_im U_mc) V_cc.
// The sum is formed transposed, sum U_mc^T V_im^T, whose accumulator holds
// the sum itself in the A-operand layout of the final product with V_cc.
__device__ __forceinline__ void v_block(const double* P, double* Q, int i, int c) {
    const int l = threadIdx.x & 63, li = l & 15, lk = l >> 4;
    doublex4 t = zero4();
    for (int m = i; m < c; ++m) mm16(t, P, SB * m, SB * c, true, Q, SB * i, SB * m, false, true);
    doublex4 v = zero4();
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
        v = __builtin_amdgcn_mfma_f64_16x16x4f64(-t[kc], Q[(SB * c + 4 * kc + lk) * LD + SB * c + li], v, 0, 0, 0);
    store16(v, Q, SB * i, SB * c);
}

// Cholesky P = U^T U and V = U^-1 of the 64 x 64 diagonal block in LDS
// (upper triangle of P read; V written to Q with zeros below the diagonal;
// P is left holding U in its upper blocks and scratch below).  Recursive in
// 16-row strips: wave s factors strip s in registers (no block barrier per
// pivot), then all waves subtract the strip's product from the trailing
// 16 x 16 blocks on the matrix cores.  Each strip's wave also inverts its
// 16 x 16 diagonal block as it factors it; while strip s is factored, the
// other waves form block column s - 1 of V from the columns before it, and
// the last column follows the last strip.  Returns the 1-based column
// of the first pivot that is not positive or not finite, or 0 (in every
// thread).
__device__ int factor_diagonal(double* P, double* Q, PanelScratch& S) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), j = threadIdx.x & 63;
    static_assert(NS == 4 && NT == 256, "one wave per strip");
    // zero Q's six 16 x 16 blocks below the diagonal (no branches)
    {
        const int r = threadIdx.x >> 4, c = threadIdx.x & 15;
        constexpr int lower[6][2] = {{1, 0}, {2, 0}, {2, 1}, {3, 0}, {3, 1}, {3, 2}};
#pragma unroll
        for (int q = 0; q < 6; ++q) Q[(SB * lower[q][0] + r) * LD + SB * lower[q][1] + c] = 0.0;
    }
    __syncthreads();
    double u[SB];
#pragma unroll 1
    for (int s = 0; s < NS; ++s) {
        if (w == s) {
            const int col = (SB * s + j) & (B - 1);
#pragma unroll
            for (int c = 0; c < SB; ++c) u[c] = P[(SB * s + c) * LD + col];
            double x[SB];
            const int f = strip_factor(u, x, S, s, j);
#pragma unroll
            for (int c = 0; c < SB; ++c) P[(SB * s + c) * LD + col] = u[c];
            // row j % 16 of V_ss into the diagonal block (s, s) of Q; the four
            // lanes of a row store the same values (no branch: behind one,
            // the compiler would defer the eliminations to the store and
            // keep every pivot row live until then)
#pragma unroll
            for (int c = 0; c < SB; ++c) Q[(SB * s + (j & (SB - 1))) * LD + SB * s + c] = x[c];
            if (j == 0) S.fail[s] = f;
        } else if (w + 1 < s) {
            v_block(P, Q, w, s - 1);   // column s - 1 of V, beside strip s
        }
        __syncthreads();
        if (s + 1 < NS) {
            // trailing blocks (b, c), s < b <= c, numbered row by row
            const int n = (NS - 1 - s) * (NS - s) / 2;
            for (int q = w; q < n; q += NT / 64) {
                int b = s + 1, r = q;
                while (r >= NS - b) {
                    r -= NS - b;
                    ++b;
                }
                const int c = b + r;
                doublex4 acc;
                load16(acc, P, SB * b, SB * c);
                mm16(acc, P, SB * s, SB * b, true, P, SB * s, SB * c, true);
                store16(acc, P, SB * b, SB * c);
            }
            __syncthreads();
        }
    }
    // the last column of V
    if (w + 1 < NS) v_block(P, Q, w, NS - 1);
    __syncthreads();
    // strips are factored in order, so the first failure is the smallest code
    int f = 0;
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        const int v = S.fail[q];
        f = (v != 0 && (f == 0 || v < f)) ? v : f;
    }
    return f;
}

__device__ __forceinline__ void record_info(const InvMat& M, int k, int f) {
    if (threadIdx.x != 0) return;
    if (k == 0) {
        *as_global(M.info) = f;
    } else if (f && *as_global(M.info) == 0) {
        *as_global(M.info) = k * B + f;
    }
}

// -------------------------------------------------------------- kernels --

// W = sym(X) + gamma I on the upper blocks of the leading n x n part,
// identity in the padding.
__global__ __launch_bounds__(NT) void inv_prepare_kernel(InvLaunch L, int64_t tiles) {
    int mi;
    int64_t local;
    if (!locate(L, kInvPrepare, xcd_remap(blockIdx.x, gridDim.x), mi, local)) return;
    const InvMat M = L.mats[mi];
    int bi, bj;
    upper_decode(local, M.nb, bi, bj);
    const int64_t D = (int64_t)M.nb * B, d = M.d, n = M.n;
    const int r0 = threadIdx.x >> 6, c = threadIdx.x & 63;
    float xv[PER];
#pragma unroll
    for (int s = 0; s < PER; ++s) {
        const int64_t i = (int64_t)bi * B + r0 + 4 * s, j = (int64_t)bj * B + c;
        xv[s] = (i < n && j < n && j >= i) ? as_global(M.x)[i * d + j] : 0.0f;
    }
#pragma unroll
    for (int s = 0; s < PER; ++s) {
        const int64_t i = (int64_t)bi * B + r0 + 4 * s, j = (int64_t)bj * B + c;
        double v;
        if (i < n && j < n) {
            v = (double)xv[s];
            if (i == j) v += L.gamma;
        } else {
            v = (i == j) ? 1.0 : 0.0;  // identity padding
        }
        as_global(M.w)[i * D + j] = v;
    }
}

// Step k of potrf, row k.  The workgroup of block (k, j) first applies step
// k-1's update to the diagonal block (k, k) and to its own block, then
// factors the diagonal block and inverts its triangle (every row-k
// workgroup of a matrix does so redundantly, so no launch boundary separates
// the two), and solves U_kj = U_kk^-T W_kj.  With rowq > 1 a workgroup
// owns rowq consecutive blocks of the row and solves each of them after one
// factorisation.  The workgroup of the first such block (or of the diagonal
// alone, in a matrix's last step) stores U_kk^-1 and the failure code.
// Diagonal blocks of W are not written: later steps read dinv.
__device__ __forceinline__ void potrf_row_block(const InvLaunch& L, const InvMat& M, int64_t local, double* As,
                                                double* Bs, PanelScratch& R) {
    const int k = L.step;
    const int64_t D = (int64_t)M.nb * B;
    const bool has_right = k + 1 < M.nb;
    // this workgroup's blocks of row k right of the diagonal: [J, Jend)
    const int J = k + 1 + (int)local * L.rowq;
    const int Jend = min(J + L.rowq, M.nb);
    double* Wkk = M.w + (int64_t)k * B * D + (int64_t)k * B;
    double* Wkj = M.w + (int64_t)k * B * D + (int64_t)J * B;
    // Blocks after the first (rowq > 1): each takes the panels [plo, k) in
    // turn and is written back; its solve, after the factorisation, reads it
    // again (the same threads read the elements they wrote).
    for (int Jx = J + 1; Jx < Jend && L.rplo < k; ++Jx) {
        double* Wkx = M.w + (int64_t)k * B * D + (int64_t)Jx * B;
        doublex4 wx[2][2];
        double xa[PER], xb[PER];
        acc_load(wx, Wkx, D);
        for (int p = L.rplo; p < k; ++p) {
            fetch(xa, Blk{M.w + (int64_t)p * B * D + (int64_t)k * B, D, true});
            fetch(xb, Blk{M.w + (int64_t)p * B * D + (int64_t)Jx * B, D, true});
            put(As, xa, true);
            put(Bs, xb, true);
            __syncthreads();
            mma_block(wx, As, Bs, true);
            __syncthreads();
        }
        acc_store(wx, Wkx, D);
    }
    // Row k still lacks the updates of panels [rplo, k) (at most
    // kMaxPassDepth; one where the step before updated this row).  Every block this
    // workgroup reads first is requested before the first wait, the first
    // panel's blocks first.  The requests are unconditional (a branch around
    // them would end in a wait for all of them): without a block right of
    // the diagonal, or at step 0, they read blocks of the matrix that are
    // then not used.
    const int Jr = has_right ? J : k;
    const int p0 = L.rplo < k ? L.rplo : 0;
    double ra[PER], rb[PER];
    fetch(ra, Blk{M.w + (int64_t)p0 * B * D + (int64_t)k * B, D, true});
    fetch(rb, Blk{M.w + (int64_t)p0 * B * D + (int64_t)Jr * B, D, true});
    doublex4 dk[2][2], wj[2][2];
    acc_load(dk, Wkk, D);
    acc_load(wj, M.w + (int64_t)k * B * D + (int64_t)Jr * B, D);
    auto update = [&]() {
        put(As, ra, true);
        if (has_right) put(Bs, rb, true);
        __syncthreads();
        mma_block(dk, As, As, true);
        if (has_right) mma_block(wj, As, Bs, true);
        __syncthreads();
    };
    if (p0 < k) update();
#pragma unroll
    for (int u = 1; u < kMaxPassDepth; ++u) {   // the host keeps k - rplo <= kMaxPassDepth
        if (p0 + u < k) {
            fetch(ra, Blk{M.w + (int64_t)(p0 + u) * B * D + (int64_t)k * B, D, true});
            fetch(rb, Blk{M.w + (int64_t)(p0 + u) * B * D + (int64_t)Jr * B, D, true});
            update();
        }
    }
    acc_to_lds(dk, Bs);
    const int f = factor_diagonal(Bs, As, R);   // As: U_kk^-1
    if (local == 0) {
        const int r0 = threadIdx.x >> 6, c = threadIdx.x & 63;
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int r = r0 + 4 * s;
            as_global(M.dinv)[(int64_t)k * BB + r * B + c] = As[r * LD + c];
        }
        record_info(M, k, f);
    }
    if (!has_right) return;
    {
        const int r0 = threadIdx.x >> 6, c = threadIdx.x & 63;
        double q[PER];
#pragma unroll
        for (int s = 0; s < PER; ++s) q[s] = As[(r0 + 4 * s) * LD + c];
        __syncthreads();
        put(As, q, true);
        for_acc([&](int a, int b, int r, int row, int col) { Bs[col * LD + row] = wj[a][b][r]; });
    }
    __syncthreads();
    doublex4 acc[2][2];
    acc_zero(acc);
    mma_block(acc, As, Bs, false);
    acc_store(acc, Wkj, D);
    // the same solve for the other blocks of this workgroup
    for (int Jx = J + 1; Jx < Jend; ++Jx) {
        double* Wkx = M.w + (int64_t)k * B * D + (int64_t)Jx * B;
        doublex4 wx[2][2];
        acc_load(wx, Wkx, D);
        __syncthreads();   // the previous product is done with Bs
        for_acc([&](int a, int b, int r, int row, int col) { Bs[col * LD + row] = wx[a][b][r]; });
        __syncthreads();
        acc_zero(acc);
        mma_block(acc, As, Bs, false);
        acc_store(acc, Wkx, D);
    }
}

// Block V_im of V = U^-1 (m >= i) staged as [row][k]: the inverted diagonal
// block, or block (m, i) below the diagonal of W, which holds V_im.
__device__ __forceinline__ Blk v_low(const InvMat& M, int64_t D, int i, int m) {
    return m == i ? Blk{M.dinv + (int64_t)i * BB, B, false} : Blk{M.w + (int64_t)m * B * D + (int64_t)i * B, D, false};
}

// Partial sum of column c = step - 1 of V, slot `local`: chunk q of row i,
// sum_{m in chunk} V_im U_mc over m in [i + q kVChunk, min(i + (q + 1) kVChunk, c - 1)).
__device__ __forceinline__ void v_partial(const InvLaunch& L, const InvMat& M, int64_t local, const Stage& S) {
    const int c = L.step - 1;
    const int64_t D = (int64_t)M.nb * B;
    int q = 0;
    int64_t r = local;
    while (r >= c - 1 - (int64_t)q * kVChunk) {
        r -= c - 1 - (int64_t)q * kVChunk;
        ++q;
    }
    const int i = (int)r;
    const int m0 = i + q * kVChunk, m1 = min(m0 + kVChunk, c - 1);
    doublex4 acc[2][2];
    acc_zero(acc);
    block_gemm(acc, S, m0, m1, [&](int m) { return v_low(M, D, i, m); },
               [&](int m) { return Blk{M.w + (int64_t)m * B * D + (int64_t)c * B, D, true}; }, false, false);
    double* dst = M.part + ((int64_t)(c & 1) * vpart_slots(M.nb - 1) + local) * BB;
    acc_store(acc, dst, B);
}

// Block (i, c) of V, c = step - 2: T = (its partial blocks) + V_i,c-1 U_c-1,c,
// then V_ic = -T V_cc, stored into block (c, i) of W (below the diagonal).
__device__ __forceinline__ void v_finalize(const InvLaunch& L, const InvMat& M, int64_t local, const Stage& S) {
    const int c = L.step - 2, i = (int)local;
    const int64_t D = (int64_t)M.nb * B;
    double* As = S.s0;
    double* Bs = S.s1;
    doublex4 acc[2][2];
    acc_zero(acc);
    const int nq = i <= c - 2 ? (c - 1 - i + kVChunk - 1) / kVChunk : 0;
    const double* part = M.part + (int64_t)(c & 1) * vpart_slots(M.nb - 1) * BB;
    // four partial blocks in flight per round trip (in chunk order, so the
    // sum is the same on every run); past nq, block 0 is read and not used
    for (int q = 0; q < nq; q += 4) {
        doublex4 t[4][2][2];
#pragma unroll
        for (int u = 0; u < 4; ++u) acc_load(t[u], part + (vpart_slot0(c, q + u < nq ? q + u : 0) + i) * BB, B);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    if (q + u < nq) acc[a][b] += t[u][a][b];
    }
    block_gemm(acc, S, c - 1, c, [&](int m) { return v_low(M, D, i, m); },
               [&](int m) { return Blk{M.w + (int64_t)m * B * D + (int64_t)c * B, D, true}; }, false, false);
    // -T V_cc: T staged as [m][k], V_cc as [n][k] = V_cc[k][n]
    double vc[PER];
    fetch(vc, Blk{M.dinv + (int64_t)c * BB, B, false});
    acc_to_lds(acc, As);
    put(Bs, vc, true);
    __syncthreads();
    doublex4 out[2][2];
    acc_zero(out);
    mma_block(out, As, Bs, true);
    acc_store(out, M.w + (int64_t)c * B * D + (int64_t)i * B, D);
}

// Step k of potrf with a look-ahead of one step.  Workgroups [0, split) are
// the row-k blocks of every matrix, the critical path: they come first in
// the dispatch and keep its order, so the hardware spreads them over the
// XCDs.  Workgroups from tail_first (a multiple of 8, so that the XCD of a
// workgroup is still its index mod 8) apply step k-1's update
// W_ij -= U_{k-1,i}^T U_{k-1,j} to the blocks k < i <= j, XCD by XCD.
__global__ __launch_bounds__(NT, 2) void inv_step_kernel(InvLaunch L, int64_t tiles) {
    __shared__ PanelScratch R;
    __shared__ __attribute__((aligned(16))) double S0[SLOT], S1[SLOT];
    const Stage S{S0, S1};
    double* As = S0;
    double* Bs = S1;
    int mi;
    int64_t local;
    const int64_t b = blockIdx.x;
    if (b < L.split) {
        if (!locate(L, kInvPanel, b, mi, local)) return;
        potrf_row_block(L, L.mats[mi], local, As, Bs, R);
        return;
    }
    if (b < L.fin_end) {
        if (!locate(L, kInvVFin, b - L.split, mi, local)) return;
        v_finalize(L, L.mats[mi], local, S);
        return;
    }
    if (b < L.part_end) {
        if (!locate(L, kInvVPart, b - L.fin_end, mi, local)) return;
        v_partial(L, L.mats[mi], local, S);
        return;
    }
    if (b < L.next_end) {
        // block (k + 1, J) of the next row takes panels [plo, k) now, off the
        // chain, so that its row workgroups at step k + 1 apply only panel k
        if (!locate(L, kInvNextRow, b - L.part_end, mi, local)) return;
        const InvMat M = L.mats[mi];
        const int k = L.step, I = k + 1, J = k + 1 + (int)local;
        const int64_t D = (int64_t)M.nb * B;
        double* Wij = M.w + (int64_t)I * B * D + (int64_t)J * B;
        doublex4 acc[2][2];
        acc_load(acc, Wij, D);
        block_gemm(acc, S, L.plo, k, [&](int t) { return Blk{M.w + (int64_t)t * B * D + (int64_t)I * B, D, true}; },
                   [&](int t) { return Blk{M.w + (int64_t)t * B * D + (int64_t)J * B, D, true}; }, true, I == J);
        acc_store(acc, Wij, D);
        return;
    }
    if (b < L.tail_first) return;
    const int64_t item = xcd_remap(b - L.tail_first, (int64_t)gridDim.x - L.tail_first);
    if (!locate(L, kInvSyrk, item, mi, local)) return;
    const InvMat M = L.mats[mi];
    const int k = L.step;
    const int T = M.nb - k - 1;
    int a, c;
    upper_decode(local, T, a, c);
    const int I = k + 1 + a, J = k + 1 + c;
    const int64_t D = (int64_t)M.nb * B;
    double* Wij = M.w + (int64_t)I * B * D + (int64_t)J * B;
    doublex4 acc[2][2];
    if (L.plo == k - 1) {
        // one 64-deep product: both panel blocks and the block being updated
        // are requested at once (a single memory round trip), then
        // multiplied from LDS
        const double* prev = M.w + (int64_t)(k - 1) * B * D;
        double ra[PER], rb[PER];
        fetch(ra, Blk{prev + (int64_t)I * B, D, true});
        if (I != J) fetch(rb, Blk{prev + (int64_t)J * B, D, true});
        acc_load(acc, Wij, D);
        put(As, ra, true);
        if (I != J) put(Bs, rb, true);
        __syncthreads();
        mma_block(acc, As, I == J ? As : Bs, true);
    } else {
        // panels [plo, k) at once: the block is read and written once for all
        acc_load(acc, Wij, D);
        block_gemm(acc, S, L.plo, k, [&](int t) { return Blk{M.w + (int64_t)t * B * D + (int64_t)I * B, D, true}; },
                   [&](int t) { return Blk{M.w + (int64_t)t * B * D + (int64_t)J * B, D, true}; }, true, I == J);
    }
    acc_store(acc, Wij, D);
}

// Slot `local` of trtri launch `step` (0 = bottom) of a matrix of nb blocks.
// Groups of 2^l blocks: level l = step + 1 joins G1 = [m*2h, m*2h + h) and
// G2 = [m*2h + h, min(m*2h + 2h, nb)), h = 2^step.  Balanced tree (nb just
// above a power of two): depth d = D - 1 - step, node n covers
// [n nb / 2^d, (n + 1) nb / 2^d) and joins its children G1 = [lo, mid),
// G2 = [mid, hi) in s2 x s2 slots, of which those beyond |G1| x |G2| have
// no work.  The slot is block (I, J), I in G1, J in G2, in row-major order,
// or with `desc_j` column by column from the last column of G2 (the longest
// products of the first trtri launch first).
__device__ __forceinline__ bool trtri_decode(int64_t local, int nb, int step, int& I, int& J, int& g1_end,
                                             bool desc_j) {
    if (trtri_balanced(nb)) {
        int D = 0;
        while ((1 << D) < nb) ++D;
        const int d = D - 1 - step;
        const int s2 = (nb + (1 << (d + 1)) - 1) >> (d + 1);
        const int n = (int)(local / ((int64_t)s2 * s2));
        const int r = (int)(local % ((int64_t)s2 * s2));
        const int bi = desc_j ? r % s2 : r / s2;
        const int bj = desc_j ? s2 - 1 - r / s2 : r % s2;
        const int lo = (int)(((int64_t)n * nb) >> d);
        const int mid = (int)(((int64_t)(2 * n + 1) * nb) >> (d + 1));
        const int hi = (int)(((int64_t)(n + 1) * nb) >> d);
        if (bi >= mid - lo || bj >= hi - mid) return false;
        I = lo + bi;
        J = mid + bj;
        g1_end = mid;
        return true;
    }
    const int h = 1 << step, g = 2 * h;
    const int full = nb / g;
    const int64_t hh = (int64_t)h * h;
    int m, bi, bj;
    if (local / hh < full) {
        m = (int)(local / hh);
        const int r = (int)(local % hh);
        bi = desc_j ? r % h : r / h;
        bj = desc_j ? h - 1 - r / h : r % h;
    } else {
        m = full;
        const int r = (int)(local - (int64_t)full * hh);
        const int w2 = nb % g - h;
        bi = desc_j ? r % h : r / w2;
        bj = desc_j ? w2 - 1 - r / h : r % w2;
    }
    I = m * g + bi;
    J = m * g + h + bj;
    g1_end = m * g + h;
    return true;
}

constexpr int KT = 16;   // k-columns per staged piece in the triangular-inverse products

// The trailing update of a step as a launch of its own: quarters of 16
// k-columns (32 KB of staging) and few registers, so four workgroups share a
// CU, against two for the step kernel.
__global__ __launch_bounds__(NT, 4) void inv_trail_kernel(InvLaunch L, int64_t tiles) {
    __shared__ __attribute__((aligned(16))) double S0[2 * B * KT], S1[2 * B * KT];
    const Stage S{S0, S1};
    int mi;
    int64_t local;
    const int64_t item = xcd_remap(blockIdx.x, gridDim.x);
    if (!locate(L, kInvSyrk, item, mi, local)) return;
    const InvMat M = L.mats[mi];
    const int k = L.step;
    const int T = M.nb - k - 1;
    int a, c;
    upper_decode(local, T, a, c);
    const int I = k + 1 + a, J = k + 1 + c;
    const int64_t D = (int64_t)M.nb * B;
    double* Wij = M.w + (int64_t)I * B * D + (int64_t)J * B;
    doublex4 acc[2][2];
    acc_load(acc, Wij, D);
    block_gemm<KT>(acc, S, L.plo, k, [&](int t) { return Blk{M.w + (int64_t)t * B * D + (int64_t)I * B, D, true}; },
                   [&](int t) { return Blk{M.w + (int64_t)t * B * D + (int64_t)J * B, D, true}; }, true, I == J);
    acc_store(acc, Wij, D);
}

// T_IJ = sum_{t in G2, t <= J} U_It V_tJ, parked in W's lower block (J, I).
__global__ __launch_bounds__(NT, 4) void inv_trtri_a_kernel(InvLaunch L, int64_t tiles) {
    // quarters of 16 k-columns (a 32 KB staging area): four workgroups share a CU
    __shared__ __attribute__((aligned(16))) double S0[2 * B * KT], S1[2 * B * KT];
    const Stage S{S0, S1};
    int mi;
    int64_t local;
    const int64_t item = xcd_runs<kRun>(blockIdx.x);
    if (item >= tiles || !locate(L, kInvTrtri, item, mi, local)) return;
    const InvMat M = L.mats[mi];
    int I, J, g1_end;
    if (!trtri_decode(local, M.nb, L.step, I, J, g1_end, true)) return;
    const int64_t D = (int64_t)M.nb * B;
    doublex4 acc[2][2];
    acc_zero(acc);
    block_gemm<KT>(acc, S, g1_end, J + 1,
               [&](int t) { return Blk{M.w + (int64_t)I * B * D + (int64_t)t * B, D, false}; },   // U_It
               [&](int t) {                                                                     // V_tJ
                   return t == J ? Blk{M.dinv + (int64_t)J * BB, B, true}
                                 : Blk{M.w + (int64_t)t * B * D + (int64_t)J * B, D, true};
               },
               false, false);
    acc_store(acc, M.w + (int64_t)J * B * D + (int64_t)I * B, D);
}

// V_IJ = - sum_{t in G1, t >= I} V_It T_tJ, written over U_IJ.
__global__ __launch_bounds__(NT, 4) void inv_trtri_b_kernel(InvLaunch L, int64_t tiles) {
    // quarters of 16 k-columns (a 32 KB staging area): four workgroups share a CU
    __shared__ __attribute__((aligned(16))) double S0[2 * B * KT], S1[2 * B * KT];
    const Stage S{S0, S1};
    int mi;
    int64_t local;
    const int64_t item = xcd_runs<kRun>(blockIdx.x);
    if (item >= tiles || !locate(L, kInvTrtri, item, mi, local)) return;
    const InvMat M = L.mats[mi];
    int I, J, g1_end;
    if (!trtri_decode(local, M.nb, L.step, I, J, g1_end, false)) return;
    const int64_t D = (int64_t)M.nb * B;
    doublex4 acc[2][2];
    acc_zero(acc);
    block_gemm<KT>(acc, S, I, g1_end,
               [&](int t) {                                                                     // V_It
                   return t == I ? Blk{M.dinv + (int64_t)I * BB, B, false}
                                 : Blk{M.w + (int64_t)I * B * D + (int64_t)t * B, D, false};
               },
               [&](int t) { return Blk{M.w + (int64_t)J * B * D + (int64_t)t * B, D, true}; },   // T_tJ at (J, t)
               true, false);
    acc_store(acc, M.w + (int64_t)I * B * D + (int64_t)J * B, D);
}

// V^T in float32 for the last product Z = V V^T, which runs on the GEMM of
// the factor stage (float32 products, K range of a tile from max(row,
// column), both triangles written).  Its error against ||Z||_F does not grow
// with the condition number: | |V| |V|^T | <= ||V||_F^2 = trace(Z) <=
// sqrt(n) ||Z||_F, so products with float32 rounding keep Z within
// float32-level error of the float64 result; the factorisation and V stay
// in float64, where errors are amplified.  One workgroup per upper block
// (I, t) of V (t >= I): the block is read row by row, rounded, transposed
// through LDS and written as rows t 64 .. of vt (columns I 64 ..); a
// diagonal block keeps only its upper triangle (rows k < i of vt are
// zero).  For odd I the block (I - 1, I) of vt, which a 128-row tile of the
// product reads, is written as zeros; for a bordered matrix the border
// column of V becomes row n.
__global__ __launch_bounds__(NT) void inv_vt32_kernel(InvLaunch L, int64_t tiles) {
    __shared__ float T[B][B + 1];
    int mi;
    int64_t local;
    if ((int64_t)blockIdx.x >= tiles || !locate(L, kInvUpper, blockIdx.x, mi, local)) return;
    const InvMat M = L.mats[mi];
    int I, t;
    column_decode(local, I, t);
    const int64_t D = (int64_t)M.nb * B, n = M.n;
    const Blk src = t == I ? Blk{M.dinv + (int64_t)I * BB, B, false}
                           : (L.vlow ? Blk{M.w + (int64_t)t * B * D + (int64_t)I * B, D, false}
                                     : Blk{M.w + (int64_t)I * B * D + (int64_t)t * B, D, false});
    double v[PER];
    fetch(v, src);
    const int r0 = threadIdx.x >> 6, c = threadIdx.x & 63;
#pragma unroll
    for (int s = 0; s < PER; ++s) {
        const int r = r0 + 4 * s;   // row i = I 64 + r of V, column k = t 64 + c
        T[c][r] = (t == I && c < r) ? 0.0f : (float)v[s];
    }
    __syncthreads();
    float* const vt = M.vt;
#pragma unroll
    for (int s = 0; s < PER; ++s) {
        const int kk = r0 + 4 * s;   // row k = t 64 + kk of vt, column i = I 64 + c
        const int64_t k = (int64_t)t * B + kk, i = (int64_t)I * B + c;
        if (k < n && i < n) as_global(vt)[k * D + i] = T[kk][c];
    }
    if (t == I) {
        if (I & 1) {
#pragma unroll
            for (int s = 0; s < PER; ++s) {
                const int64_t k = (int64_t)(I - 1) * B + r0 + 4 * s, i = (int64_t)I * B + c;
                if (i < n) as_global(vt)[k * D + i] = 0.0f;
            }
        }
        if (n < M.d && threadIdx.x < B) {
            const int64_t i = (int64_t)I * B + threadIdx.x;
            if (i < n) as_global(vt)[n * D + i] = (float)as_global(M.bvec)[i];
        }
    }
}

// Block (row, t) of V = U^-1 in whichever place it is kept: above the
// diagonal, or in block (t, row) below it when formed beside potrf; the
// diagonal blocks in dinv.
__device__ __forceinline__ Blk v_blk(const InvLaunch& L, const InvMat& M, int64_t D, int row, int t) {
    if (L.vlow) return v_low(M, D, row, t);
    return t == row ? Blk{M.dinv + (int64_t)row * BB, B, false}
                    : Blk{M.w + (int64_t)row * B * D + (int64_t)t * B, D, false};
}

// The last row and column of a bordered matrix (order d = n + 1, leading
// n x n part already factored, Y_11 = U^T U, V = U^-1), as one more step of
// the Cholesky factorisation: with x the last column above the diagonal and
// xi = x_nn + gamma, the factor of the whole matrix has the column
// w = U^-T x = V^T x and the pivot mu = sqrt(xi - w^T w), and its inverse
// the column v = -V w / mu and the pivot 1 / mu.  Three launches, each
// workgroup summing a run of kBorderRun blocks, partial sums kept in the
// matrix's border workspace and added in a fixed order.
//
// w: workgroup (matrix, c, q) sums V_ic^T x_i over i in run q of
// [0, c], i = q kBorderRun + u.
__global__ __launch_bounds__(NT) void inv_border_w_kernel(InvLaunch L, int64_t tiles) {
    static_assert(NT == 4 * B && kBorderRun == 4, "four row groups of a block, one x value per thread and run");
    __shared__ double xs[kBorderRun * B];
    __shared__ double red[4][B];
    int mi;
    int64_t local;
    if (blockIdx.x >= tiles || !locate(L, kInvBorderRun, blockIdx.x, mi, local)) return;
    const InvMat M = L.mats[mi];
    const int64_t runs = border_runs(M.nb);
    const int c = (int)(local / runs), q = (int)(local % runs);
    const int i0 = q * kBorderRun;
    if (M.n == M.d || i0 > c) return;
    const int64_t D = (int64_t)M.nb * B, d = M.d, n = M.n;
    const int j = threadIdx.x & 63, g = threadIdx.x >> 6;
    {
        const int64_t row = (int64_t)i0 * B + threadIdx.x;   // < (c + 1) B <= n when kept
        xs[threadIdx.x] = row < (int64_t)(c + 1) * B ? (double)as_global(M.x)[row * d + n] : 0.0;
    }
    double vv[kBorderRun][PER];
#pragma unroll
    for (int u = 0; u < kBorderRun; ++u) {
        const int i = i0 + u <= c ? i0 + u : c;
        const Blk b = v_blk(L, M, D, i, c);
#pragma unroll
        for (int s = 0; s < PER; ++s) vv[u][s] = as_global(b.p)[(int64_t)(g + 4 * s) * b.ld + j];
    }
    __syncthreads();
    double acc = 0.0;
#pragma unroll
    for (int u = 0; u < kBorderRun; ++u) {
        double t = 0.0;
#pragma unroll
        for (int s = 0; s < PER; ++s) t += vv[u][s] * xs[u * B + g + 4 * s];
        acc += i0 + u <= c ? t : 0.0;
    }
    red[g][j] = acc;
    __syncthreads();
    if (g == 0)
        as_global(M.bvec)[border_w_off(M.nb) + ((int64_t)c * runs + q) * B + j] =
            red[0][j] + red[1][j] + red[2][j] + red[3][j];
}

// u = V w: workgroup (matrix, i, q) first completes w_c (its partials, in
// run order) for c in run q of [i, nb), c = i + q kBorderRun + u, then sums
// V_ic w_c.  The workgroups of row 0 cover every c once and also sum w^T w
// over their run.
__global__ __launch_bounds__(NT) void inv_border_u_kernel(InvLaunch L, int64_t tiles) {
    __shared__ double red[B][B + 1];
    int mi;
    int64_t local;
    if (blockIdx.x >= tiles || !locate(L, kInvBorderRun, blockIdx.x, mi, local)) return;
    const InvMat M = L.mats[mi];
    const int64_t runs = border_runs(M.nb);
    const int i = (int)(local / runs), q = (int)(local % runs);
    const int c0 = i + q * kBorderRun;
    if (M.n == M.d || c0 >= M.nb) return;
    const int64_t D = (int64_t)M.nb * B;
    const double* wp = M.bvec + border_w_off(M.nb);
    const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;
    double vv[kBorderRun][PER], wc[kBorderRun];
#pragma unroll
    for (int u = 0; u < kBorderRun; ++u) {
        const int c = c0 + u < M.nb ? c0 + u : M.nb - 1;
        const Blk b = v_blk(L, M, D, i, c);
#pragma unroll
        for (int s = 0; s < PER; ++s) vv[u][s] = as_global(b.p)[(int64_t)(g + 4 * s) * b.ld + lane];
        double w = 0.0;
        const int nq = (int)border_runs(c + 1);
        for (int qq = 0; qq < nq; ++qq) w += as_global(wp)[((int64_t)c * runs + qq) * B + lane];
        wc[u] = c0 + u < M.nb ? w : 0.0;
    }
    double acc[PER];
#pragma unroll
    for (int s = 0; s < PER; ++s) {
        acc[s] = 0.0;
#pragma unroll
        for (int u = 0; u < kBorderRun; ++u) acc[s] += vv[u][s] * wc[u];
    }
#pragma unroll
    for (int s = 0; s < PER; ++s) red[g + 4 * s][lane] = acc[s];
    if (i == 0 && g == 0) {
        double ss = 0.0;
#pragma unroll
        for (int u = 0; u < kBorderRun; ++u) ss += wc[u] * wc[u];
        for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
        if (lane == 0) as_global(M.bvec)[border_ss_off(M.nb) + q] = ss;
    }
    __syncthreads();
    if (threadIdx.x < B) {
        const int r = threadIdx.x;
        double u = 0.0;
        for (int j = 0; j < B; ++j) u += red[r][j];
        as_global(M.bvec)[border_u_off(M.nb) + ((int64_t)i * runs + q) * B + r] = u;
    }
}

// v: workgroup (matrix, i) completes u_i (its partials, in run order) and
// w^T w, stores v_i = -u_i / mu for the product V V^T, and writes the border
// of the inverse, z_rn = z_nr = v_r / mu and z_nn = 1 / mu^2.  A pivot mu^2
// that is not positive and finite is reported as info = d, unless the
// leading part has failed already.
__global__ __launch_bounds__(NT) void inv_border_v_kernel(InvLaunch L, int64_t tiles) {
    int mi;
    int64_t local;
    if (blockIdx.x >= tiles || !locate(L, kInvBorder, blockIdx.x, mi, local)) return;
    const InvMat M = L.mats[mi];
    if (M.n == M.d || threadIdx.x >= B) return;
    const int i = (int)local, r = threadIdx.x;
    const int64_t d = M.d, n = M.n, runs = border_runs(M.nb);
    double ss = 0.0;
    for (int q = 0; q < runs; ++q) ss += as_global(M.bvec)[border_ss_off(M.nb) + q];
    double u = 0.0;
    const int nq = (int)border_runs(M.nb - i);
    for (int q = 0; q < nq; ++q) u += as_global(M.bvec)[border_u_off(M.nb) + ((int64_t)i * runs + q) * B + r];
    const double xi = (double)as_global(M.x)[n * d + n] + L.gamma;
    const double mu2 = xi - ss;
    const double mu = sqrt(mu2);
    const double v = -u / mu;
    const int64_t row = (int64_t)i * B + r;
    as_global(M.bvec)[row] = v;
    const float zb = (float)(v / mu);
    as_global(M.z)[row * d + n] = zb;
    as_global(M.z)[n * d + row] = zb;
    if (i == 0 && r == 0) {
        as_global(M.z)[n * d + n] = (float)(1.0 / mu2);
        if (!(mu2 > 0.0 && isfinite(mu2)) && *as_global(M.info) == 0) *as_global(M.info) = (int32_t)d;
    }
}

template <typename K>
hipError_t launch(K kernel, const InvLaunch& L, int64_t tiles, hipStream_t s, bool runs = false) {
    if (tiles <= 0) return hipSuccess;
    const int64_t grid = runs ? (tiles + 8 * kRun - 1) / (8 * kRun) * (8 * kRun) : tiles;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(NT), 0, s, L, tiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_inv_prepare(const InvLaunch& L, int64_t t, hipStream_t s) { return launch(inv_prepare_kernel, L, t, s); }
hipError_t launch_inv_step(const InvLaunch& L, int64_t t, hipStream_t s) { return launch(inv_step_kernel, L, t, s); }
hipError_t launch_inv_trail(const InvLaunch& L, int64_t t, hipStream_t s) { return launch(inv_trail_kernel, L, t, s); }
hipError_t launch_inv_trtri_a(const InvLaunch& L, int64_t t, hipStream_t s) { return launch(inv_trtri_a_kernel, L, t, s, true); }
hipError_t launch_inv_trtri_b(const InvLaunch& L, int64_t t, hipStream_t s) { return launch(inv_trtri_b_kernel, L, t, s, true); }
hipError_t launch_inv_vt32(const InvLaunch& L, int64_t t, hipStream_t s) { return launch(inv_vt32_kernel, L, t, s); }
hipError_t launch_inv_border_w(const InvLaunch& L, int64_t t, hipStream_t s) { return launch(inv_border_w_kernel, L, t, s); }
hipError_t launch_inv_border_u(const InvLaunch& L, int64_t t, hipStream_t s) { return launch(inv_border_u_kernel, L, t, s); }
hipError_t launch_inv_border_v(const InvLaunch& L, int64_t t, hipStream_t s) { return launch(inv_border_v_kernel, L, t, s); }

}  // namespace kfac
