// Internal declarations shared by the host launchers and the kernels of the
// K-FAC library.  Nothing here is part of the public ABI (include/kfac.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kfac {

// ----------------------------------------------------------------- tables --
// Per-call descriptor tables live in the caller's workspace.  They are
// written by a tiny kernel whose by-value argument carries the bytes, so the
// upload is ordered on the stream like every other launch, needs no pinned
// host memory, and survives stream capture.
constexpr int kTableChunk = 2048;
struct TableChunk {
    uint8_t bytes[kTableChunk];
};
hipError_t upload_table(void* dst_device, const void* src_host, size_t nbytes, hipStream_t stream);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// --------------------------------------------------------- fp32 MFMA GEMM --
// C = alpha * Aop^T Bop with Aop [K][lda] and Bop [K][ldb] row-major (the
// reduction index is the slow index of both operands).  Used for
//   factors:        Aop = Bop = X [rows][d], upper tiles only, running average;
//   precondition:   S^T = grad^T Z_G  (Aop = grad, Bop = Z_G)  and
//                   P   = (S^T)^T Z_A (Aop = S^T,  Bop = Z_A).
constexpr int kGemmTile = 128;     // output tile edge (BM = BN)
constexpr int kGemmBK = 32;        // rows of each operand staged per LDS buffer
constexpr int kGemmThreads = 256;  // 4 waves, 2 x 2 over the tile, 64 x 64 each
constexpr int kGemmSubK = 512;     // rows accumulated before folding into the running sum

// Wide bfloat16 factor tiles: 256 rows x 128 columns per workgroup, each wave
// 128 x 64.  For factor launches with bf16 inputs whose rows all start on a
// 4-byte boundary, no problem split along K, and at most kWideMaxK rows: the
// products go into one float32 sum per element without the second-level
// fold (at most kWideMaxK / 16 additions of exact 16-term products).
constexpr int kWideM = 256;
constexpr int kWideN = 128;
constexpr int kWideMaxK = 16384;
constexpr int64_t kWideMinTiles = 1024;   // fewer tiles than this leave CUs idle: 128 x 128 tiles instead

// The wide tiles of a factor of order d: tile row I (rows 256 I ..) holds the
// tile columns J >= 2 I (columns 128 J ..), the ones that reach the upper
// triangle.  Tiles are numbered in bands of two tile rows, column by
// column: band b has row 2 b from column 4 b and row 2 b + 1 from column
// 4 b + 2 (each row holds at least one tile).
__host__ __device__ inline int64_t wide_band_tiles(int64_t b, int64_t ti, int64_t tj) {
    return (tj - 4 * b) + (2 * b + 1 < ti ? tj - 4 * b - 2 : 0);
}
__host__ __device__ inline int64_t wide_tiles(int64_t d) {
    const int64_t ti = (d + kWideM - 1) / kWideM, tj = (d + kWideN - 1) / kWideN;
    int64_t n = 0;
    for (int64_t b = 0; 2 * b < ti; ++b) n += wide_band_tiles(b, ti, tj);
    return n;
}

enum GemmMode : int32_t { kModePlain = 0, kModeFactor = 1 };
// GemmProb flags: the K range of an output tile starts at max(first row,
// first column) (an operand that is zero above its diagonal, Aop[k][i] = 0
// for k < i), and every element kept is also written to its mirror position.
enum GemmFlag : int32_t { kGemmTriK = 1, kGemmMirror = 2 };

struct GemmProb {
    const void* a;        // Aop
    const void* b;        // Bop (== a for factors)
    float* c;             // output (factor: running-average matrix M)
    float* part;          // split-K partial tiles (nullptr when ksplit == 1)
    int64_t lda, ldb, ldc;
    int64_t item_begin;   // first work item of this problem in the GEMM launch
    int64_t red_begin;    // first tile of this problem in the split-K reduce launch
    int32_t M, N, K;
    int32_t tiles_m, tiles_n;
    int32_t ntiles;       // output tiles (upper tiles only for factors)
    int32_t ksplit;       // K chunks
    int32_t kchunk;       // rows per chunk, multiple of kGemmBK
    int32_t mode;         // GemmMode
    int32_t bf16;         // operands are bfloat16 bit patterns
    float alpha;
    int32_t flags;        // GemmFlag bits
};

struct GemmLaunch {
    const GemmProb* probs;
    int32_t nprob;
    int32_t first_step;
    float eps;
    int32_t runs;         // set by the launchers: items go to XCDs in runs (large launches)
    int32_t tile;         // output tile edge of the launch (kGemmTile)
};

// C = alpha Aop^T Bop on 128 x 128 tiles (float32 operands, or bfloat16
// operands when `bf16`), then, for split K, the partials summed in chunk
// order and the epilogue.  `factor` picks the kernel names of the factor
// stage (else those of the preconditioning products); `bf16_aligned` says
// that every bf16 operand row starts on a 4-byte boundary, `bf16_edges`
// that some problem's order is not a multiple of the tile edge.
hipError_t launch_gemm(const GemmLaunch& L, int64_t items, hipStream_t stream, bool bf16, bool factor,
                       bool bf16_aligned = true, bool bf16_edges = true);
hipError_t launch_gemm_reduce(const GemmLaunch& L, int64_t tiles, hipStream_t stream, bool factor);
// bf16 factors on wide tiles (problems numbered by wide_tiles, K unsplit);
// `edges`: some order is not a multiple of 256.
hipError_t launch_factor_wide(const GemmLaunch& L, int64_t items, hipStream_t stream, bool edges);

// An odd-width bf16 input copied to a pitch that is a multiple of 64 elements
// (rows start on 128-byte lines; columns past d zero); 256 groups of 8
// elements per workgroup.
struct RepackLayer {
    const uint16_t* src;   // [rows][d]
    uint16_t* dst;         // [rows][pitch], 256-byte aligned
    int64_t rows;
    int64_t block_begin;   // first workgroup of this layer
    int32_t d, pitch;
};
__host__ __device__ inline int64_t repack_pitch(int64_t d) { return (d + 63) / 64 * 64; }
hipError_t launch_repack_bf16(const RepackLayer* layers, int n, int64_t blocks, hipStream_t stream);

// ----------------------------------------------------------------- layers --
constexpr int kLayerTile = 64;       // im2col and gradient-row tiles are 64 x 64
constexpr int kGradMatChunk = 4096;  // elements per workgroup in kfac_grad_matrix

struct Im2colLayer {
    const void* x;
    void* a;
    int64_t c, h, w;
    int64_t rows;         // n * oh * ow
    int64_t tile_begin;   // first work item of this layer
    int32_t kh, kw, sh, sw, ph, pw, dh, dw;
    int32_t oh, ow;
    int32_t cols;         // c * kh * kw + ones
    int32_t ones;
    int32_t tiles_c;      // column tiles
    int32_t vec;          // kVecIn | kVecOut
};

// Four-element accesses of the layer kernels: kVecIn when every group of
// four consecutive rows of a tile is four consecutive, aligned elements of
// the input, kVecOut when the rows of the output hold a multiple of four
// elements and start aligned.
constexpr int32_t kVecIn = 1, kVecOut = 2;

struct GradRowsLayer {
    const void* gy;
    void* g;
    int64_t batch, c, hw;
    int64_t tile_begin;
    int32_t tiles_c;      // channel tiles
    int32_t tiles_p;      // position tiles per sample (hw > 1) or batch tiles (hw == 1)
    int32_t vec;          // kVecIn | kVecOut
    int32_t pad_;
};

struct GradMatLayer {
    float* w;
    float* b;
    float* mat;
    int64_t d_out, d_in;
    int64_t chunk_begin;
    int64_t cols;         // d_in + (b != nullptr)
};

hipError_t launch_im2col(const Im2colLayer* layers, int n, int64_t tiles, bool bf16, hipStream_t stream);
hipError_t launch_grad_rows(const GradRowsLayer* layers, int n, int64_t tiles, bool bf16, float scale,
                            hipStream_t stream);
hipError_t launch_grad_matrix(const GradMatLayer* layers, int n, int64_t chunks, bool pack, hipStream_t stream);

// ------------------------------------------------------------------- pack --
// The host uploads (pointer, order) per factor; one wavefront on the device
// turns them into the layer table, whose offsets are exclusive prefix sums of
// d (d + 1) / 2 (packed elements) and of T (T + 1) / 2, T = ceil(d / 64)
// (unpack tiles).
struct PackSrc {
    float* m;
    int64_t d;
};
struct PackLayer {
    float* m;             // [d][d] matrix
    int64_t d;
    int64_t off;          // first packed element of this layer
    int64_t tile_begin;   // first unpack tile of this layer
    int64_t tiles_1d;     // unpack tiles per edge
};
constexpr int kUnpackTile = 64;
constexpr int kPackThreads = 256;
constexpr int kPackUnits = 2;    // 16-byte units per pack thread: 2048 packed elements per workgroup
hipError_t launch_pack_table(const PackSrc* src, int n, PackLayer* out, hipStream_t stream);
hipError_t launch_pack(const PackLayer* layers, int n, float* packed, int64_t total, hipStream_t stream);
hipError_t launch_unpack(const PackLayer* layers, int n, const float* packed, int64_t tiles, hipStream_t stream);
// Device copy of `bytes` (a multiple of 16, both pointers 16-byte aligned),
// one 16-byte unit per lane: the streaming reference for the pack figures.
hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

// ---------------------------------------------------------------- inverse --
// Every matrix is padded with the identity to D = NB * kInvNB and factored in
// float64 in the workspace.  Matrices are grouped in buckets of equal NB,
// largest first; each blocked step launches over all matrices that still
// have work at that step.
constexpr int kInvNB = 64;
constexpr int kInvThreads = 256;

struct InvMat {
    const float* x;       // input (upper read), [d][d]
    float* z;             // output, [d][d]
    double* w;            // workspace [D][D] float64: U, then V = U^-1 above the diagonal
    double* dinv;         // workspace [NB][64][64]: inverses of the diagonal blocks of U
    int32_t* info;        // &info[original index]
    double* part;         // workspace: partial blocks of V, 2 x vpart_slots(nb - 1) blocks (by column parity)
    double* bvec;         // bordered matrices (n < d): border_doubles(nb), see there
    float* vt;            // workspace [n + 1][64 nb] float32: V^T, and for a bordered matrix the
                          // border column of V as row n; the operand of the last product Z = V V^T
    int32_t d;            // order of the matrix and row stride of x and z
    int32_t n;            // order of the part factored in blocks: d, or d - 1 when the last row and
                          // column are attached afterwards as a border
    int32_t nb;           // blocks per edge, ceil(n / 64)
    int32_t pad_;
};

// Order of the part of a d x d matrix that is factored in 64 x 64 blocks.
// A matrix one larger than a multiple of 64 (the factor A of a layer with a
// bias) would waste a whole block row and column on its last index, so that
// index is attached after the inverse of the leading part, through its Schur
// complement (a bordered Cholesky step).
__host__ __device__ inline int64_t inv_extent(int64_t d) { return (d > kInvNB && d % kInvNB == 1) ? d - 1 : d; }

// Workspace of a bordered matrix, in doubles: the border column v of V
// (n = 64 nb), the partial sums of w^T w (one per run of columns, padded to
// 64), then the partial sums of w (per column block and run of row blocks)
// and of u = V w (per row block and run of column blocks), 64 each.  A run
// is kBorderRun blocks, the share of one workgroup.
constexpr int kBorderRun = 4;
__host__ __device__ inline int64_t border_runs(int64_t nb) { return (nb + kBorderRun - 1) / kBorderRun; }
__host__ __device__ inline int64_t border_ss_off(int64_t nb) { return nb * kInvNB; }
__host__ __device__ inline int64_t border_w_off(int64_t nb) {
    return border_ss_off(nb) + (border_runs(nb) + kInvNB - 1) / kInvNB * kInvNB;
}
__host__ __device__ inline int64_t border_u_off(int64_t nb) { return border_w_off(nb) + nb * border_runs(nb) * kInvNB; }
__host__ __device__ inline int64_t border_doubles(int64_t nb) { return border_u_off(nb) + nb * border_runs(nb) * kInvNB; }

struct InvBucket {
    int32_t nb;           // blocks per edge of every matrix in the bucket
    int32_t first;        // first matrix (index into the sorted InvMat table)
    int32_t count;        // matrices in the bucket
    int32_t pad_;
};

struct InvLaunch {
    const InvMat* mats;
    const InvBucket* buckets;
    int32_t nbuckets;
    int32_t step;         // k for potrf steps, level for trtri
    double gamma;
    int64_t split;        // potrf step launch: blocks [0, split) are row-k blocks
    int64_t tail_first;   // potrf step launch: first block of the trailing update
    int64_t fin_end;      // potrf step launch: [split, fin_end) finish a column of V
    int64_t part_end;     // potrf step launch: [fin_end, part_end) partial sums of the next column
    int32_t vlow;         // V_ic is kept in block (c, i) below the diagonal (formed beside potrf), not in (i, c)
    int32_t plo;          // potrf step launch: the trailing update (and the next row) apply panels [plo, k)
    int32_t rowq;         // potrf step launch: blocks of row k per row workgroup (>= 1)
    int32_t rplo;         // potrf step launch: row k applies panels [rplo, k)
    int64_t next_end;     // potrf step launch: [part_end, next_end) update row k + 1 with panels [plo, k)
};
// At most this many panels per trailing update (k - plo).
constexpr int kMaxPassDepth = 3;

// Tiles each inverse kernel needs per matrix with nb blocks per edge at a
// given potrf step (trsm, syrk) or trtri level.  Shared by the host, which
// sizes the grids, and the kernels, which decode their tile index.
enum InvKind : int32_t {
    kInvPrepare = 0, kInvPanel = 1, kInvSyrk = 2, kInvTrtri = 3, kInvUpper = 4,
    kInvVPart = 6, kInvVFin = 7, kInvBorder = 8, kInvBorderRun = 9, kInvNextRow = 10
};

// V = U^-1 formed column by column beside the potrf steps (V U = I):
//   V_ic = -(sum_{i <= m < c} V_im U_mc) V_cc,  i < c.
// Step launch k sums, for column c = k - 1, the terms m <= c - 2 in chunks of
// kVChunk blocks (one partial block per chunk and row i), and finishes column
// c = k - 2: its partial blocks, the term m = c - 1, and the product with V_cc.
// Partial slots of a column: chunk q covers rows i <= c - 2 - q kVChunk, so
// chunk q holds c - 1 - q kVChunk slots, chunk by chunk.
constexpr int kVChunk = 2;
__host__ __device__ inline int64_t vpart_slot0(int64_t c, int64_t q) {   // first slot of chunk q
    return q * (c - 1) - (int64_t)kVChunk * q * (q - 1) / 2;
}
__host__ __device__ inline int64_t vpart_slots(int64_t c) {
    if (c < 2) return 0;
    const int64_t nq = (c - 1 + kVChunk - 1) / kVChunk;
    return vpart_slot0(c, nq);
}

// Groups of 2^l blocks leave a last level that joins almost all blocks with
// a handful when nb is just above a power of two (33 = 32 + 1): a few long
// products on a nearly idle chip.  Such matrices use a balanced binary tree.
__host__ __device__ inline bool trtri_balanced(int64_t nb) {
    int64_t p = 1;
    while (2 * p < nb) p *= 2;          // p < nb <= 2p
    return nb > 2 && nb - p <= p / 8;
}

__host__ __device__ inline int64_t inv_tiles(int kind, int64_t nb, int64_t step, int64_t rowq = 1) {
    switch (kind) {
        case kInvPrepare:
        case kInvUpper:
            return nb * (nb + 1) / 2;
        case kInvVPart: {  // partial sums of column step - 1
            const int64_t c = step - 1;
            return c >= 2 && c < nb ? vpart_slots(c) : 0;
        }
        case kInvVFin: {   // rows 0 .. c - 1 of column c = step - 2
            const int64_t c = step - 2;
            return c >= 1 && c < nb ? c : 0;
        }
        case kInvBorder:  // one workgroup per block row of the leading part
            return nb;
        case kInvBorderRun:  // one workgroup per block row (or column) and run of blocks
            return nb * border_runs(nb);
        case kInvPanel: {  // one workgroup per rowq blocks right of the diagonal, at least one
            const int64_t right = nb - step - 1;
            return nb > step ? (right > rowq ? (right + rowq - 1) / rowq : 1) : 0;
        }
        case kInvNextRow:  // the blocks (k + 1, j), j >= k + 1
            return step + 1 < nb ? nb - step - 1 : 0;
        case kInvSyrk: {  // step k applies step k-1's update to blocks (i, j), k < i <= j
            const int64_t t = nb - step - 1;
            return step >= 1 && t > 0 ? t * (t + 1) / 2 : 0;
        }
        case kInvTrtri: {
            // launch `step` (0 = bottom) serves level step + 1 of groups of
            // 2^l blocks, or, for nb just above a power of two, depth
            // D - 1 - step of the balanced tree (D = ceil(log2 nb))
            int D = 0;
            while ((int64_t(1) << D) < nb) ++D;
            if (step >= D) return 0;
            if (trtri_balanced(nb)) {
                const int d = D - 1 - (int)step;
                const int64_t s2 = (nb + (int64_t(1) << (d + 1)) - 1) >> (d + 1);
                return (int64_t(1) << d) * s2 * s2;
            }
            const int64_t h = int64_t(1) << step, g = 2 * h;
            const int64_t full = nb / g, rem = nb % g;
            return full * h * h + (rem > h ? h * (rem - h) : 0);
        }
        default:
            return 0;
    }
}

hipError_t launch_inv_prepare(const InvLaunch& L, int64_t tiles, hipStream_t s);
hipError_t launch_inv_step(const InvLaunch& L, int64_t tiles, hipStream_t s);
hipError_t launch_inv_trail(const InvLaunch& L, int64_t tiles, hipStream_t stream);
hipError_t launch_inv_trtri_a(const InvLaunch& L, int64_t tiles, hipStream_t s);
hipError_t launch_inv_trtri_b(const InvLaunch& L, int64_t tiles, hipStream_t s);
hipError_t launch_inv_vt32(const InvLaunch& L, int64_t tiles, hipStream_t s);
hipError_t launch_inv_border_w(const InvLaunch& L, int64_t tiles, hipStream_t s);
hipError_t launch_inv_border_u(const InvLaunch& L, int64_t tiles, hipStream_t s);
hipError_t launch_inv_border_v(const InvLaunch& L, int64_t tiles, hipStream_t s);

}  // namespace kfac
