// MFMA GEMMs for the factor (syrk, upper tiles, running average) and
// precondition (two plain products) stages.
//
// C = alpha * Aop^T Bop, Aop [K][lda], Bop [K][ldb], both with the reduction
// index as the slow (row) index, so every staged K-slab is a set of
// contiguous row segments and the global loads coalesce.
//
// Tile 128 x 128 per workgroup of 4 waves (2 x 2, 64 x 64 each, four
// accumulators per wave).  Products are summed in float32 over sub-chunks
// of kGemmSubK rows and then folded into a second float32 sum, which keeps
// the rounding error of long reductions (hundreds of thousands of rows)
// near that of a 512-term sum.  Operands are read with buffer loads whose
// descriptor covers one K-slab: rows past the end of the input read as
// zero without a branch, and the per-thread offsets inside a slab are
// computed once.
//
// float32 operands run on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16,
// 16 times the rate of v_mfma_f32_32x32x2f32 on gfx950): every value is
// split exactly into three bf16 values and each block product becomes six
// bf16 products, which carry the rounding of a float32 product (see the
// split kernel below).  bfloat16 inputs go from memory straight into LDS as
// [k][m] rows and are read back with transposing LDS reads, since
// v_mfma_f32_32x32x16_bf16 takes 8 consecutive k-values per lane; rows of
// odd width are first repacked to an aligned pitch (bf16_repack.hip), and
// only an input of even width at a base one element off a 4-byte boundary
// passes through registers, stored as [m][k].  bf16 factor launches with K
// unsplit, at most kWideMaxK rows and enough tiles take 256 x 128 tiles
// (each wave 128 x 64), which read fewer LDS bytes per product.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace kfac {
namespace {

constexpr int BM = kGemmTile;
constexpr int BK = kGemmBK;
constexpr int NT = kGemmThreads;
constexpr int kGemmRun = 16;        // items per XCD run in large launches
constexpr int64_t kGemmRunsMin = 2048;

__device__ __forceinline__ int find_prob(const GemmProb* probs, int nprob, int64_t item, bool reduce) {
    int lo = 0, hi = nprob - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        const int64_t begin = reduce ? probs[mid].red_begin : probs[mid].item_begin;
        if (begin <= item) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Epilogue of one output element (row i, column j of the problem): kept
// when inside the problem (and on or above the diagonal for a factor), with
// `prev` the element's value before the call.
__device__ __forceinline__ bool elem_kept(const GemmProb& P, int i, int j) {
    return i < P.M && j < P.N && (P.mode != kModeFactor || j >= i);
}
__device__ __forceinline__ float elem_value(const GemmProb& P, float v, float prev, float eps, int first) {
    if (P.mode != kModeFactor) return v * P.alpha;
    const float f = v * P.alpha;
    return first ? f : eps * prev + (1.0f - eps) * f;
}
// The old value for the running average, read from element 0 when (i, j)
// is not kept, so the read needs no branch.
__device__ __forceinline__ float elem_prev(const GemmProb& P, int i, int j) {
    const int64_t off = elem_kept(P, i, j) ? (int64_t)i * P.ldc + j : 0;
    return as_global(P.c)[off];
}
__device__ __forceinline__ void elem_store(const GemmProb& P, int i, int j, float r) {
    if (elem_kept(P, i, j)) {
        as_global(P.c)[(int64_t)i * P.ldc + j] = r;
        if ((P.flags & kGemmMirror) && j != i) as_global(P.c)[(int64_t)j * P.ldc + i] = r;
    }
}

constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past any slab: loads return 0

// Buffer resource over rows [k0, min(k0 + BK, k_end)) of a row-major
// operand; rows past the end of the slab read as zero.
// The range ends at column `cols` of the slab's last row (the operand's
// last element there), not at the end of that row: a 16-byte copy that
// straddles the last column then stops at the operand's end instead of
// reading past it.  The range is checked per dword, so it is rounded up to
// a 4-byte boundary: otherwise a last bf16 element sharing its dword with
// the next (a row of odd width repacked to an even pitch) would read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const void* base, int64_t ld, int k0, int k_end, int esz,
                                                            int cols) {
    const char* p = static_cast<const char*>(base) + (int64_t)k0 * ld * esz;
    const int rows = max(0, min(BK, k_end - k0));
    // every operand is uniform; readfirstlane keeps the descriptor in
    // scalar registers (a per-lane descriptor would need a waterfall loop)
    const int bytes = __builtin_amdgcn_readfirstlane(rows > 0 ? (((rows - 1) * (int)ld + cols) * esz + 3) & ~3 : 0);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0, bytes, 0x00020000);
}

// Writes a finished 128 x 128 tile: to the split-K partial buffer when K is
// split, else through the epilogue.  Output layout of a 32 x 32 MFMA block:
// lane l holds column (l % 32); register r holds row 8*(r/4) + 4*(l/32) + (r%4).
// The running average reads every old value of the thread's 64 elements,
// then forms every result, then writes: with the reads, or the stores'
// inputs, behind per-element branches, each store would wait for the
// memory operations before it.
__device__ __forceinline__ void store_tile(const GemmProb& P, const GemmLaunch& L, const floatx16 (&sum)[2][2],
                                           int kc, int t, int m0, int n0, int wm, int wn, int lane) {
    const int khalf = lane >> 5;
    auto row_of = [&](int a, int r) { return wm * 64 + a * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3); };
    auto col_of = [&](int b) { return wn * 64 + b * 32 + (lane & 31); };
    if (P.ksplit > 1) {
        float* part = P.part + ((int64_t)kc * P.ntiles + t) * (BM * BM);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) as_global(part)[row_of(a, r) * BM + col_of(b)] = sum[a][b][r];
        return;
    }
    floatx16 res[2][2];
    if (P.mode == kModeFactor && !L.first_step) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) res[a][b][r] = elem_prev(P, m0 + row_of(a, r), n0 + col_of(b));
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) res[a][b][r] = elem_value(P, sum[a][b][r], res[a][b][r], L.eps, L.first_step);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) elem_store(P, m0 + row_of(a, r), n0 + col_of(b), res[a][b][r]);
}

// Tiles are numbered in bands of kBand tile rows, column by column within a
// band, so that kBand^2 consecutive tiles form about a kBand x kBand block.
// Large launches hand the XCDs runs of kGemmRun = kBand^2 consecutive items,
// so the tiles of a run read 2 kBand operand panels between them, which the
// XCD's L2 serves to all of them (in row order, a run of tiles in one tile
// row reads one panel of A and a different panel of B per tile).  Factor
// problems number only the upper triangle (i <= j); there the first kBand
// columns of a band form a triangle.
constexpr int kBand = 4;
static_assert(kBand * kBand == kGemmRun, "an XCD run is one block of tiles");
__device__ __forceinline__ void tile_decode(const GemmProb& P, int64_t t, int& ti, int& tj) {
    if (P.flags & kGemmTriK) {
        // K runs from the tile's column on: column by column, the longest first
        column_decode(t, ti, tj);
    } else if (P.mode == kModeFactor) {
        upper_band_decode(t, P.tiles_m, kBand, ti, tj);
    } else {
        const int64_t i0 = t / ((int64_t)kBand * P.tiles_n) * kBand;
        const int64_t r = min<int64_t>(kBand, P.tiles_m - i0);
        const int64_t u = t - i0 * P.tiles_n;
        ti = (int)(i0 + u % r);
        tj = (int)(u / r);
    }
}

// Tile and K-chunk of a work item.
struct TileWork {
    GemmProb P;
    int kc, t, m0, n0, k_begin, k_end;
    bool same, active;
};

__device__ __forceinline__ TileWork decode_item(const GemmLaunch& L, int64_t item) {
    TileWork w;
    w.P = L.probs[find_prob(L.probs, L.nprob, item, false)];
    const GemmProb& P = w.P;
    const int64_t q = item - P.item_begin;
    w.kc = (int)(q / P.ntiles);
    w.t = (int)(q % P.ntiles);
    int ti, tj;
    tile_decode(P, w.t, ti, tj);
    w.m0 = ti * BM;
    w.n0 = tj * BM;
    w.k_begin = w.kc * P.kchunk;
    w.k_end = min(P.K, w.k_begin + P.kchunk);
    // an operand zero above its diagonal contributes from row max(m0, n0) on
    if (P.flags & kGemmTriK) w.k_begin = max(w.k_begin, max(w.m0, w.n0));
    // factor tiles on the diagonal read the same columns for both operands
    w.same = (P.a == P.b) && (w.m0 == w.n0);
    const int wave = threadIdx.x >> 6;
    // the wave below the diagonal of a diagonal factor tile has nothing to compute
    w.active = !(P.mode == kModeFactor && ti == tj && (wave >> 1) > (wave & 1));
    return w;
}

// bfloat16 inputs on v_mfma_f32_32x32x16_bf16 (products exact in float32,
// float32 accumulation).  Slabs of 32 rows are staged as [m][k] bf16 with k
// contiguous; a lane's eight k-values of a block are one 16-byte LDS read,
// and each slab feeds 2 x 4 MFMAs per wave.  This path loads elements one
// at a time and serves rows that are not 4-byte aligned (odd width), which
// the 16-byte copies into LDS cannot read.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr int BK16 = 32;
constexpr int LDK16 = BK16 + 8;    // LDS row stride in bf16 (80 bytes)
constexpr int LOADS16 = BK16 * BM / NT;   // 16 rows of one column per thread

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc16(const void* base, int64_t ld, int k0, int k_end) {
    const char* p = static_cast<const char*>(base) + (int64_t)k0 * ld * 2;
    const int rows = max(0, min(BK16, k_end - k0));
    const int bytes = __builtin_amdgcn_readfirstlane(rows * (int)ld * 2);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ void gemm_bf16_reg_tile(const GemmLaunch& L, const TileWork& W,
                                                   uint16_t (&As)[2][BM * LDK16], uint16_t (&Bs)[2][BM * LDK16]) {
    const GemmProb& P = W.P;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // thread t loads column lc, slab rows lr16 .. lr16+15
    const int lc = tid & (BM - 1);
    const int lr16 = (tid >> 7) * LOADS16;
    uint32_t offa[LOADS16], offb[LOADS16];
#pragma unroll
    for (int s = 0; s < LOADS16; ++s) {
        const int row = lr16 + s;
        offa[s] = (W.m0 + lc < P.M) ? (uint32_t)((row * P.lda + W.m0 + lc) * 2) : kOOB;
        offb[s] = (W.n0 + lc < P.N) ? (uint32_t)((row * P.ldb + W.n0 + lc) * 2) : kOOB;
    }
    uint16_t ra[LOADS16], rb[LOADS16];
    auto gload = [&](int k0) {
        const __amdgpu_buffer_rsrc_t rA = slab_rsrc16(P.a, P.lda, k0, W.k_end);
#pragma unroll
        for (int s = 0; s < LOADS16; ++s) ra[s] = __builtin_amdgcn_raw_buffer_load_b16(rA, offa[s], 0, 0);
        if (!W.same) {
            const __amdgpu_buffer_rsrc_t rB = slab_rsrc16(P.b, P.ldb, k0, W.k_end);
#pragma unroll
            for (int s = 0; s < LOADS16; ++s) rb[s] = __builtin_amdgcn_raw_buffer_load_b16(rB, offb[s], 0, 0);
        }
    };
    auto pack8 = [](const uint16_t* v) {
        uint4 u;
        u.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
        u.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
        u.z = (uint32_t)v[4] | ((uint32_t)v[5] << 16);
        u.w = (uint32_t)v[6] | ((uint32_t)v[7] << 16);
        return u;
    };
    auto sstore = [&](int buf) {
        uint4* da = reinterpret_cast<uint4*>(&As[buf][lc * LDK16 + lr16]);
        da[0] = pack8(ra);
        da[1] = pack8(ra + 8);
        if (!W.same) {
            uint4* db = reinterpret_cast<uint4*>(&Bs[buf][lc * LDK16 + lr16]);
            db[0] = pack8(rb);
            db[1] = pack8(rb + 8);
        }
    };

    floatx16 acc[2][2], sum[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) { acc[a][b][r] = 0.0f; sum[a][b][r] = 0.0f; }

    const int nstages = (W.k_end - W.k_begin + BK16 - 1) / BK16;
    if (nstages > 0) {
        gload(W.k_begin);
        sstore(0);
    }
    __syncthreads();

    // lane l supplies rows/columns (l % 32) of its blocks; MFMA step s of a
    // slab takes slab rows 16 s + 8 (l / 32) + 0..7
    const int fr = lane & 31;
    const int fk = (lane >> 5) * 8;
    constexpr int SUB16 = kGemmSubK / BK16;

    for (int st = 0; st < nstages; ++st) {
        const int buf = st & 1;
        if (st + 1 < nstages) gload(W.k_begin + (st + 1) * BK16);
        if (W.active) {
            const uint16_t* Ab = As[buf];
            const uint16_t* Bb = W.same ? As[buf] : Bs[buf];
#pragma unroll
            for (int s = 0; s < BK16 / 16; ++s) {
                bf16x8 fa[2], fb[2];
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    fa[a] = *reinterpret_cast<const bf16x8*>(&Ab[(wm * 64 + a * 32 + fr) * LDK16 + 16 * s + fk]);
                    fb[a] = *reinterpret_cast<const bf16x8*>(&Bb[(wn * 64 + a * 32 + fr) * LDK16 + 16 * s + fk]);
                }
                acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[0], fb[0], acc[0][0], 0, 0, 0);
                acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[0], fb[1], acc[0][1], 0, 0, 0);
                acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[1], fb[0], acc[1][0], 0, 0, 0);
                acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[1], fb[1], acc[1][1], 0, 0, 0);
            }
            if ((st + 1) % SUB16 == 0 || st + 1 == nstages) {
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        sum[a][b] += acc[a][b];
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
                    }
            }
        }
        if (st + 1 < nstages) sstore(buf ^ 1);
        __syncthreads();
    }
    store_tile(P, L, sum, W.kc, W.t, W.m0, W.n0, wm, wn, lane);
}

// bfloat16 slabs are copied straight into LDS as [k][m] (16 bytes, 8
// columns, per lane).  The matrix cores take 8 consecutive k-values per
// lane; two transposing LDS reads (ds_read_b64_tr_b16) assemble them: in a
// group of 16 lanes, lane p points at k-row k0 + p/4, columns mb + 4 (p % 4),
// and lane i receives column mb + i of rows k0 .. k0 + 3.  The 16-byte chunks
// of row k sit at position c xor swz(k % 4), swz = 0, 6, 12, 10: the two
// groups of a half-wave read chunks c0 .. c0 + 3 (c0 a multiple of 4) of
// four consecutive rows, which then fall on four disjoint quarters of a
// 256-byte bank line (bits 2-3 of the position differ), and each group's
// two chunks per row on four disjoint quarters of a 128-byte line (bits
// 1-2 differ).  With c xor 2 (k % 4) the rows paired up on the same banks
// (half of the LDS cycles were conflicts).
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef short short8v __attribute__((ext_vector_type(8)));
constexpr int SLAB16 = BK16 * BM;                  // bf16 per staged slab (8 KB)
constexpr int kSlab16Copies = SLAB16 / (8 * NT);   // copy instructions per wave and slab (2)
static_assert(kSlab16Copies * 8 * NT == SLAB16, "a slab is a whole number of 16-byte copies per lane");

__device__ __forceinline__ int tr_swz(int k) {
    const int x = k & 3;
    return (2 * x) ^ (4 * x);
}
__device__ __forceinline__ int tr_at(int k, int m) {
    return k * BM + ((((m >> 3) ^ tr_swz(k)) << 3) | (m & 7));
}

__device__ __forceinline__ void stage_slab16(uint16_t* S, __amdgpu_buffer_rsrc_t r,
                                             const uint32_t (&off)[kSlab16Copies]) {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int s = 0; s < kSlab16Copies; ++s)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(S + 512 * (kSlab16Copies * w + s)), 16, off[s], 0, 0, 0);
}

// The products of a full wave, with the LDS reads written out, for the ring below.  The
// compiler, which cannot follow which ring buffer each copy in flight
// targets across the loop, would otherwise wait for every copy before the
// reads of one of the buffers.  It then also does not track these reads,
// so the waits before the products that use them are explicit: the reads
// of step 0 and the A fragments of step 1 are issued, then (12 in flight)
// lgkmcnt(4) before step 0's products, the B fragments of step 1, and
// lgkmcnt(0) before step 1's.  The wait takes the fragments as operands, so
// no product moves above it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)reinterpret_cast<uintptr_t>(p); }
__device__ __forceinline__ short4v tr_read(uint32_t a) {
    short4v v;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(a));
    return v;
}
__device__ __forceinline__ void mma_slab16_ring(floatx16 (&acc)[2][2], const uint16_t* A, const uint16_t* Bm, int wm,
                                                int wn, int lane) {
    const int g = lane >> 4, p = lane & 15;
    // lane p of a group reads k-rows k0 + p/4 and k0 + 4 + p/4, columns mb + 4 (p % 4)
    auto addr = [&](const uint16_t* S, int k0, int mb) { return lds_addr(S + tr_at(k0 + (p >> 2), mb + 4 * (p & 3))); };
    auto addr_hi = [&](const uint16_t* S, int k0, int mb) {
        return lds_addr(S + tr_at(k0 + 4 + (p >> 2), mb + 4 * (p & 3)));
    };
    short4v fa[2][2][2], fb[2][2][2];   // [step][block][lo/hi]
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const int k0 = 16 * st + 8 * (g >> 1);
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const int mb = wm * 64 + a * 32 + 16 * (g & 1);
            fa[st][a][0] = tr_read(addr(A, k0, mb));
            fa[st][a][1] = tr_read(addr_hi(A, k0, mb));
        }
        if (st == 0) {
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const int nb = wn * 64 + a * 32 + 16 * (g & 1);
                fb[0][a][0] = tr_read(addr(Bm, k0, nb));
                fb[0][a][1] = tr_read(addr_hi(Bm, k0, nb));
            }
        }
    }
    asm volatile("s_waitcnt lgkmcnt(4)"
                 : "+v"(fa[0][0][0]), "+v"(fa[0][0][1]), "+v"(fa[0][1][0]), "+v"(fa[0][1][1]), "+v"(fb[0][0][0]),
                   "+v"(fb[0][0][1]), "+v"(fb[0][1][0]), "+v"(fb[0][1][1]));
    {
        const int k0 = 16 + 8 * (g >> 1);
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const int nb = wn * 64 + a * 32 + 16 * (g & 1);
            fb[1][a][0] = tr_read(addr(Bm, k0, nb));
            fb[1][a][1] = tr_read(addr_hi(Bm, k0, nb));
        }
    }
    auto frag = [](const short4v& lo, const short4v& hi) {
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        if (st == 1)
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(fa[1][0][0]), "+v"(fa[1][0][1]), "+v"(fa[1][1][0]), "+v"(fa[1][1][1]),
                           "+v"(fb[1][0][0]), "+v"(fb[1][0][1]), "+v"(fb[1][1][0]), "+v"(fb[1][1][1]));
        const bf16x8 a0 = frag(fa[st][0][0], fa[st][0][1]), a1 = frag(fa[st][1][0], fa[st][1][1]);
        const bf16x8 b0 = frag(fb[st][0][0], fb[st][0][1]), b1 = frag(fb[st][1][0], fb[st][1][1]);
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
    }
}

// The products of a wave at the edge of a problem: NA x NB of its 32 x 32
// blocks hold rows / columns of the problem (the others lie wholly past
// them and are left at zero).  Reads written out as for a full wave, with
// one wait per step (these waves are few).
template <int NA, int NB>
__device__ __forceinline__ void mma_slab16_edge(floatx16 (&acc)[2][2], const uint16_t* A, const uint16_t* Bm, int wm,
                                                int wn, int lane) {
    const int g = lane >> 4, p = lane & 15;
    auto addr = [&](const uint16_t* S, int k0, int mb) { return lds_addr(S + tr_at(k0 + (p >> 2), mb + 4 * (p & 3))); };
    auto addr_hi = [&](const uint16_t* S, int k0, int mb) {
        return lds_addr(S + tr_at(k0 + 4 + (p >> 2), mb + 4 * (p & 3)));
    };
    auto frag = [](const short4v& lo, const short4v& hi) {
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const int k0 = 16 * st + 8 * (g >> 1);
        short4v fa[2][2], fb[2][2];
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            const int mb = wm * 64 + a * 32 + 16 * (g & 1);
            fa[a][0] = tr_read(addr(A, k0, mb));
            fa[a][1] = tr_read(addr_hi(A, k0, mb));
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int nb = wn * 64 + b * 32 + 16 * (g & 1);
            fb[b][0] = tr_read(addr(Bm, k0, nb));
            fb[b][1] = tr_read(addr_hi(Bm, k0, nb));
        }
        if constexpr (NA == 2 && NB == 2)
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fa[0][0]), "+v"(fa[0][1]), "+v"(fa[1][0]), "+v"(fa[1][1]),
                         "+v"(fb[0][0]), "+v"(fb[0][1]), "+v"(fb[1][0]), "+v"(fb[1][1]));
        else if constexpr (NA == 2)
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fa[0][0]), "+v"(fa[0][1]), "+v"(fa[1][0]), "+v"(fa[1][1]),
                         "+v"(fb[0][0]), "+v"(fb[0][1]));
        else if constexpr (NB == 2)
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fa[0][0]), "+v"(fa[0][1]), "+v"(fb[0][0]), "+v"(fb[0][1]),
                         "+v"(fb[1][0]), "+v"(fb[1][1]));
        else
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fa[0][0]), "+v"(fa[0][1]), "+v"(fb[0][0]), "+v"(fb[0][1]));
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(fa[a][0], fa[a][1]), frag(fb[b][0], fb[b][1]),
                                                                    acc[a][b], 0, 0, 0);
    }
}

// Slabs in flight: at 128 x 128 bf16 tiles a slab feeds the matrix cores for
// only a few hundred cycles, less than a copy takes to arrive, so the slabs
// go through a ring of kRing16 buffers: while slab s is multiplied, the
// copies of slabs s + 1 .. s + kRing16 - 1 are in flight.
constexpr int kRing16 = 4;

// vmcnt(n) alone (expcnt and lgkmcnt left at their maximum)
__device__ __forceinline__ constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// A barrier that waits only for the workgroup's LDS accesses, so that the
// copies of later slabs stay in flight (__syncthreads() would wait for all
// of them).  The memory clobber keeps LDS accesses on their side of it.
__device__ __forceinline__ void lds_barrier16() {
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

// The ring: one LDS array per buffer (A's slab, then B's), so that the
// compiler can tell the copies into one buffer from the reads of another
// and waits for no copy it need not.
struct Ring16 {
    uint16_t* s[kRing16];
};

// EDGES: the launch has problems whose last tile row or column is partial
// (their waves run only their valid blocks); without it every wave runs all four.
template <bool SAME, bool EDGES>
__device__ __forceinline__ void gemm_bf16_lds_tile(const GemmLaunch& L, const TileWork& W, const Ring16& R) {
    const GemmProb& P = W.P;
    const int k_begin = W.k_begin, k_end = W.k_end;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // a wave whose 64 rows or columns all lie past the problem's edge has
    // nothing to compute; one whose second 32 do runs only its valid blocks
    const int wr = W.m0 + 64 * wm, wc = W.n0 + 64 * wn;
    const bool active = W.active && (!EDGES || (wr < P.M && wc < P.N));
    const bool a2 = wr + 32 < P.M, b2 = wc + 32 < P.N, full = !EDGES || (a2 && b2);
    uint32_t offa[kSlab16Copies], offb[kSlab16Copies];
#pragma unroll
    for (int s = 0; s < kSlab16Copies; ++s) {
        const int q = (kSlab16Copies * wave + s) * 64 + lane;
        const int k = q >> 4, c = (q & 15) ^ tr_swz(k), m = 8 * c;   // this copy's row and columns
        offa[s] = (W.m0 + m < P.M) ? (uint32_t)((k * P.lda + W.m0 + m) * 2) : kOOB;
        offb[s] = (W.n0 + m < P.N) ? (uint32_t)((k * P.ldb + W.n0 + m) * 2) : kOOB;
    }
    auto stage = [&](int buf, int k0) {
        stage_slab16(R.s[buf], slab_rsrc(P.a, P.lda, k0, k_end, 2, P.M), offa);
        if (!SAME) stage_slab16(R.s[buf] + SLAB16, slab_rsrc(P.b, P.ldb, k0, k_end, 2, P.N), offb);
    };
    // copy instructions of one slab, per wave
    constexpr int CPS = kSlab16Copies * (SAME ? 1 : 2);
    floatx16 acc[2][2], sum[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) { acc[a][b][r] = 0.0f; sum[a][b][r] = 0.0f; }
    constexpr int SUB16 = kGemmSubK / BK16;
    auto fold = [&](int st, int nstages) {
        if ((st + 1) % SUB16 == 0 || st + 1 == nstages) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    sum[a][b] += acc[a][b];
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
                }
        }
    };
    const int nstages = (k_end - k_begin + BK16 - 1) / BK16;
#pragma unroll
    for (int s = 0; s < kRing16 - 1; ++s)
        if (s < nstages) stage(s, k_begin + s * BK16);
    for (int st = 0; st < nstages; st += kRing16) {
#pragma unroll
        for (int r = 0; r < kRing16; ++r) {
            const int cur = st + r;
            if (cur < nstages) {
                // slab cur has arrived once no more than the copies of the
                // slabs after it that are already issued are outstanding
                const int after = min(kRing16 - 2, nstages - 1 - cur);
                static_assert(kRing16 == 4, "the waits below cover up to two later slabs");
                if (after >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * CPS));
                else if (after == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPS));
                else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                // the slab is visible to every wave, and the buffer of the
                // slab before it, which the next copies overwrite, is read
                lds_barrier16();
                if (cur + kRing16 - 1 < nstages) stage((r + kRing16 - 1) % kRing16, k_begin + (cur + kRing16 - 1) * BK16);
                if (active) {
                    const uint16_t* SA = R.s[r];
                    const uint16_t* SB = R.s[r] + (SAME ? 0 : SLAB16);
                    if (full) mma_slab16_ring(acc, SA, SB, wm, wn, lane);
                    else if (a2) mma_slab16_edge<2, 1>(acc, SA, SB, wm, wn, lane);
                    else if (b2) mma_slab16_edge<1, 2>(acc, SA, SB, wm, wn, lane);
                    else mma_slab16_edge<1, 1>(acc, SA, SB, wm, wn, lane);
                    fold(cur, nstages);
                }
            }
        }
    }
    store_tile(P, L, sum, W.kc, W.t, W.m0, W.n0, wm, wn, lane);
}

// Inputs whose rows all start 4-byte aligned (an even row pitch and an
// aligned base: after the repack, every input) take the copy path.  A launch
// with any other input uses the second kernel, which also holds the register
// path that loads elements one at a time (and, with its larger LDS, runs one
// workgroup per CU).
template <bool EDGES>
__device__ __forceinline__ void factor_bf16_item(const GemmLaunch& L, int64_t items) {
    __shared__ __attribute__((aligned(16))) uint16_t S0[2 * SLAB16];
    __shared__ __attribute__((aligned(16))) uint16_t S1[2 * SLAB16];
    __shared__ __attribute__((aligned(16))) uint16_t S2[2 * SLAB16];
    __shared__ __attribute__((aligned(16))) uint16_t S3[2 * SLAB16];
    const int64_t item = L.runs ? xcd_runs<kGemmRun>(blockIdx.x) : xcd_remap(blockIdx.x, gridDim.x);
    if (item >= items) return;
    const TileWork W = decode_item(L, item);
    const Ring16 R{{S0, S1, S2, S3}};
    if (W.same) gemm_bf16_lds_tile<true, EDGES>(L, W, R);
    else gemm_bf16_lds_tile<false, EDGES>(L, W, R);
}

// Launches whose problems all have whole tiles skip the edge tests.
__global__ __launch_bounds__(NT, 2) void factor_bf16_kernel(GemmLaunch L, int64_t items) { factor_bf16_item<false>(L, items); }
__global__ __launch_bounds__(NT, 2) void factor_bf16_edge_kernel(GemmLaunch L, int64_t items) { factor_bf16_item<true>(L, items); }

__global__ __launch_bounds__(NT, 1) void factor_bf16_any_kernel(GemmLaunch L, int64_t items) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDK16];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BM * LDK16];
    __shared__ __attribute__((aligned(16))) uint16_t S0[2 * SLAB16];
    __shared__ __attribute__((aligned(16))) uint16_t S1[2 * SLAB16];
    __shared__ __attribute__((aligned(16))) uint16_t S2[2 * SLAB16];
    __shared__ __attribute__((aligned(16))) uint16_t S3[2 * SLAB16];
    const int64_t item = L.runs ? xcd_runs<kGemmRun>(blockIdx.x) : xcd_remap(blockIdx.x, gridDim.x);
    if (item >= items) return;
    const TileWork W = decode_item(L, item);
    const GemmProb& P = W.P;
    const bool copy = ((P.lda | P.ldb) & 1) == 0 && (((uintptr_t)P.a | (uintptr_t)P.b) & 3) == 0;
    const Ring16 R{{S0, S1, S2, S3}};
    if (!copy) gemm_bf16_reg_tile(L, W, As, Bs);
    else if (W.same) gemm_bf16_lds_tile<true, true>(L, W, R);
    else gemm_bf16_lds_tile<false, true>(L, W, R);
}

// Wide bfloat16 factor tiles: 256 rows x 128 columns, each wave 128 x 64
// (4 x 2 blocks of 32 x 32).  The LDS serves about 128 bytes per clock per CU
// (a probe of the transposing reads alone sustains 116); at 128 x 128 tiles
// each product of a wave reads 1 KB of fragments and the slab copies write
// another 0.5 KB into LDS per product, which caps the matrix cores near two
// thirds of their rate.  A 128 x 64 wave reads 0.75 KB per product and the
// copies write 0.375 KB.  Slabs are staged as for the 128 x 128 tiles
// ([k][m] rows, 16-byte chunks swizzled by row): A's rows 256 columns long,
// B's 128.  A tile that reaches the diagonal (J = 2 I or 2 I + 1) stages
// only A and reads B's columns from it.  K is never split here and the sum
// is not folded (at most kWideMaxK rows).  Three slabs in a ring: with 72 KB
// of LDS and at most 256 registers per lane, two workgroups share a CU, so
// that one's epilogue overlaps the other's products.
constexpr int WM = kWideM, WN = kWideN;
constexpr int SLAB_WA = BK16 * WM;                 // bf16 per A slab (16 KB)
constexpr int SLAB_WB = BK16 * WN;                 // bf16 per B slab (8 KB)
constexpr int kWideCopiesA = SLAB_WA / (8 * NT);   // copy instructions per wave and A slab (4)
constexpr int kWideCopiesB = SLAB_WB / (8 * NT);   // and B slab (2)
constexpr int kWideRing = 3;
static_assert(kWideCopiesA * 8 * NT == SLAB_WA && kWideCopiesB * 8 * NT == SLAB_WB,
              "a slab is a whole number of 16-byte copies per lane");
static_assert(WM == 2 * WN, "a tile row spans two tile columns");

struct RingW {
    uint16_t* s[kWideRing];
};

// Position of element (k, m) in a staged slab whose rows hold LD columns.
template <int LD>
__device__ __forceinline__ int tr_at_ld(int k, int m) {
    return k * LD + ((((m >> 3) ^ tr_swz(k)) << 3) | (m & 7));
}

// Both transposing reads of the fragment of the 32-wide block at column mb:
// lane p of group g points at k-rows k0 + p/4 (lo) and k0 + 4 + p/4 (hi),
// columns mb + 16 (g % 2) + 4 (p % 4).
template <int LD>
__device__ __forceinline__ void wide_frag_read(short4v (&f)[2], const uint16_t* S, int k0, int mb, int g, int p) {
    const int m = mb + 16 * (g & 1) + 4 * (p & 3);
    f[0] = tr_read(lds_addr(S + tr_at_ld<LD>(k0 + (p >> 2), m)));
    f[1] = tr_read(lds_addr(S + tr_at_ld<LD>(k0 + 4 + (p >> 2), m)));
}

__device__ __forceinline__ bf16x8 wide_frag(const short4v (&f)[2]) {
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(f[0], f[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// The products of one slab for a whole wave (A columns am .. am + 127 of
// the A slab, B columns bn .. bn + 63 of the B slab).  At most 12 reads are
// in flight: step 0's fragments of A blocks 0-1 and B, then of A blocks
// 2-3; step 1's fragments follow as step 0's products free their turn.
// Each wait names the fragments it covers, so that no product moves above
// it.  With MASK, only the blocks whose bit (2 a + b) is set in `live` are
// multiplied (the others lie wholly below the diagonal or past the
// problem's edge; their fragments are read all the same).
template <int LDA, int LDB, bool MASK>
__device__ __forceinline__ void mma_wide(floatx16 (&acc)[4][2], const uint16_t* A, const uint16_t* B, int am, int bn,
                                         int lane, uint32_t live) {
    auto mfma = [&](int a, int b, const bf16x8& x, const bf16x8& y) {
        if (!MASK || ((live >> (2 * a + b)) & 1u))
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, acc[a][b], 0, 0, 0);
    };
    const int g = lane >> 4, p = lane & 15;
    const int k00 = 8 * (g >> 1), k01 = 16 + k00;
    short4v fa0[4][2], fb0[2][2], fa1[4][2], fb1[2][2];
    wide_frag_read<LDA>(fa0[0], A, k00, am, g, p);
    wide_frag_read<LDA>(fa0[1], A, k00, am + 32, g, p);
    wide_frag_read<LDB>(fb0[0], B, k00, bn, g, p);
    wide_frag_read<LDB>(fb0[1], B, k00, bn + 32, g, p);
    wide_frag_read<LDA>(fa0[2], A, k00, am + 64, g, p);
    wide_frag_read<LDA>(fa0[3], A, k00, am + 96, g, p);
    asm volatile("s_waitcnt lgkmcnt(4)"
                 : "+v"(fa0[0][0]), "+v"(fa0[0][1]), "+v"(fa0[1][0]), "+v"(fa0[1][1]), "+v"(fb0[0][0]),
                   "+v"(fb0[0][1]), "+v"(fb0[1][0]), "+v"(fb0[1][1]));
    wide_frag_read<LDA>(fa1[0], A, k01, am, g, p);
    wide_frag_read<LDA>(fa1[1], A, k01, am + 32, g, p);
    wide_frag_read<LDB>(fb1[0], B, k01, bn, g, p);
    wide_frag_read<LDB>(fb1[1], B, k01, bn + 32, g, p);
    const bf16x8 b00 = wide_frag(fb0[0]), b01 = wide_frag(fb0[1]);
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const bf16x8 x = wide_frag(fa0[a]);
        mfma(a, 0, x, b00);
        mfma(a, 1, x, b01);
    }
    asm volatile("s_waitcnt lgkmcnt(8)" : "+v"(fa0[2][0]), "+v"(fa0[2][1]), "+v"(fa0[3][0]), "+v"(fa0[3][1]));
    wide_frag_read<LDA>(fa1[2], A, k01, am + 64, g, p);
    wide_frag_read<LDA>(fa1[3], A, k01, am + 96, g, p);
#pragma unroll
    for (int a = 2; a < 4; ++a) {
        const bf16x8 x = wide_frag(fa0[a]);
        mfma(a, 0, x, b00);
        mfma(a, 1, x, b01);
    }
    asm volatile("s_waitcnt lgkmcnt(4)"
                 : "+v"(fa1[0][0]), "+v"(fa1[0][1]), "+v"(fa1[1][0]), "+v"(fa1[1][1]), "+v"(fb1[0][0]),
                   "+v"(fb1[0][1]), "+v"(fb1[1][0]), "+v"(fb1[1][1]));
    const bf16x8 b10 = wide_frag(fb1[0]), b11 = wide_frag(fb1[1]);
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const bf16x8 x = wide_frag(fa1[a]);
        mfma(a, 0, x, b10);
        mfma(a, 1, x, b11);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fa1[2][0]), "+v"(fa1[2][1]), "+v"(fa1[3][0]), "+v"(fa1[3][1]));
#pragma unroll
    for (int a = 2; a < 4; ++a) {
        const bf16x8 x = wide_frag(fa1[a]);
        mfma(a, 0, x, b10);
        mfma(a, 1, x, b11);
    }
}

// Tile (I, J) of wide tile t of a problem (numbering of wide_tiles).
__device__ __forceinline__ void wide_decode(int64_t t, int64_t ti, int64_t tj, int& I, int& J) {
    int64_t b = 0;
    while (2 * b + 2 < ti) {
        const int64_t n = wide_band_tiles(b, ti, tj);
        if (t < n) break;
        t -= n;
        ++b;
    }
    if (t < 2) {
        I = (int)(2 * b);
        J = (int)(4 * b + t);
    } else if (2 * b + 1 < ti) {
        I = (int)(2 * b + ((t - 2) & 1));
        J = (int)(4 * b + 2 + (t - 2) / 2);
    } else {
        I = (int)(2 * b);
        J = (int)(4 * b + t);
    }
}

// SAME: the tile reaches the diagonal (B's columns lie inside A's).
// EDGES: the launch has problems whose order is not a multiple of 256.
template <bool SAME, bool EDGES>
__device__ __forceinline__ void gemm_bf16_wide_tile(const GemmLaunch& L, const GemmProb& P, int m0, int n0,
                                                    const RingW& R) {
    const int K = P.K;
    // the wave index is uniform: in a scalar register, so that the block
    // mask below and the branches on it are scalar too
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int wr = m0 + 128 * wm, wc = n0 + 64 * wn;
    // the wave's blocks (a, b) with an element on or above the diagonal and
    // inside the problem; a wave with none has nothing to compute
    uint32_t live = 0;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int r0 = wr + 32 * a, c0 = wc + 32 * b;
            if ((!SAME || r0 <= c0 + 31) && (!EDGES || (r0 < P.M && c0 < P.N))) live |= 1u << (2 * a + b);
        }
    const bool active = live != 0;
    uint32_t offa[kWideCopiesA], offb[kWideCopiesB];
#pragma unroll
    for (int s = 0; s < kWideCopiesA; ++s) {
        const int q = (kWideCopiesA * wave + s) * 64 + lane;
        const int k = q >> 5, c = (q & 31) ^ tr_swz(k), m = 8 * c;   // this copy's row and columns
        offa[s] = (m0 + m < P.M) ? (uint32_t)((k * P.lda + m0 + m) * 2) : kOOB;
    }
#pragma unroll
    for (int s = 0; s < kWideCopiesB; ++s) {
        const int q = (kWideCopiesB * wave + s) * 64 + lane;
        const int k = q >> 4, c = (q & 15) ^ tr_swz(k), m = 8 * c;
        offb[s] = (n0 + m < P.N) ? (uint32_t)((k * P.ldb + n0 + m) * 2) : kOOB;
    }
    auto stage = [&](int buf, int k0) {
        uint16_t* S = R.s[buf];
        const __amdgpu_buffer_rsrc_t ra = slab_rsrc(P.a, P.lda, k0, K, 2, P.M);
#pragma unroll
        for (int s = 0; s < kWideCopiesA; ++s)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (__attribute__((address_space(3))) void*)(S + 512 * (kWideCopiesA * wave + s)), 16, offa[s], 0, 0,
                0);
        if (!SAME) {
            const __amdgpu_buffer_rsrc_t rb = slab_rsrc(P.b, P.ldb, k0, K, 2, P.N);
#pragma unroll
            for (int s = 0; s < kWideCopiesB; ++s)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rb, (__attribute__((address_space(3))) void*)(S + SLAB_WA + 512 * (kWideCopiesB * wave + s)), 16,
                    offb[s], 0, 0, 0);
        }
    };
    constexpr int CPS = kWideCopiesA + (SAME ? 0 : kWideCopiesB);   // copy instructions of one slab, per wave
    constexpr int LDB = SAME ? WM : WN;
    const int am = 128 * wm, bn = (SAME ? n0 - m0 : 0) + 64 * wn;
    floatx16 acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
    const int nstages = (K + BK16 - 1) / BK16;
#pragma unroll
    for (int s = 0; s < kWideRing - 1; ++s)
        if (s < nstages) stage(s, s * BK16);
    for (int st = 0; st < nstages; st += kWideRing) {
#pragma unroll
        for (int r = 0; r < kWideRing; ++r) {
            const int cur = st + r;
            if (cur < nstages) {
                // slab cur has arrived once only the next slab's copies are outstanding
                static_assert(kWideRing == 3, "one later slab in flight at the wait");
                if (cur + 1 < nstages) __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPS));
                else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                // the slab is visible to every wave, and the buffer of the
                // slab before it, which the next copies overwrite, is read
                lds_barrier16();
                if (cur + kWideRing - 1 < nstages) stage((r + kWideRing - 1) % kWideRing, (cur + kWideRing - 1) * BK16);
                if (active) {
                    const uint16_t* SA = R.s[r];
                    const uint16_t* SB = SAME ? SA : SA + SLAB_WA;
                    mma_wide<WM, LDB, SAME || EDGES>(acc, SA, SB, am, bn, lane, live);
                }
            }
        }
    }
    if (!active) return;   // every element of such a wave lies below the diagonal or past the edge
    // the epilogue in two halves of the wave's rows (64 old values in flight)
    const int khalf = lane >> 5;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        auto row_of = [&](int a, int r) { return m0 + am + (2 * h + a) * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3); };
        auto col_of = [&](int b) { return n0 + 64 * wn + b * 32 + (lane & 31); };
        floatx16 res[2][2];
        if (!L.first_step) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) res[a][b][r] = elem_prev(P, row_of(a, r), col_of(b));
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    res[a][b][r] = elem_value(P, acc[2 * h + a][b][r], res[a][b][r], L.eps, L.first_step);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) elem_store(P, row_of(a, r), col_of(b), res[a][b][r]);
    }
}

template <bool EDGES>
__device__ __forceinline__ void factor_bf16_wide_item(const GemmLaunch& L, int64_t items) {
    __shared__ __attribute__((aligned(16))) uint16_t W0[SLAB_WA + SLAB_WB];
    __shared__ __attribute__((aligned(16))) uint16_t W1[SLAB_WA + SLAB_WB];
    __shared__ __attribute__((aligned(16))) uint16_t W2[SLAB_WA + SLAB_WB];
    const int64_t item = L.runs ? xcd_runs<kGemmRun>(blockIdx.x) : xcd_remap(blockIdx.x, gridDim.x);
    if (item >= items) return;
    const GemmProb P = L.probs[find_prob(L.probs, L.nprob, item, false)];
    int I, J;
    wide_decode(item - P.item_begin, P.tiles_m, P.tiles_n, I, J);
    const RingW R{{W0, W1, W2}};
    if (J <= 2 * I + 1) gemm_bf16_wide_tile<true, EDGES>(L, P, I * WM, J * WN, R);
    else gemm_bf16_wide_tile<false, EDGES>(L, P, I * WM, J * WN, R);
}

__global__ __launch_bounds__(NT, 2) void factor_bf16_wide_kernel(GemmLaunch L, int64_t items) {
    factor_bf16_wide_item<false>(L, items);
}
__global__ __launch_bounds__(NT, 2) void factor_bf16_wide_edge_kernel(GemmLaunch L, int64_t items) {
    factor_bf16_wide_item<true>(L, items);
}

// float32 products on the bf16 matrix cores.  The float32 matrix cores of
// gfx950 run at 1/16 the rate of the bf16 ones.  A float32 value splits
// exactly into three bf16 values, x = x0 + x1 + x2: x0 = bf16(x) rounded to
// nearest, x1 = bf16(x - x0), x2 = x - x0 - x1 (each difference is exact in
// float32, and the last has at most 8 significant bits).  |x1| <= 2^-8 |x|
// and |x2| <= 2^-16 |x|, so x y is x0 y0 + x0 y1 + x1 y0 + x0 y2 + x1 y1 +
// x2 y0 up to the three dropped cross terms, below 2^-23 |x y| together and
// of either sign; each of the six products is exact in float32.  The sum
// therefore carries the rounding of a float32 product, and the six products
// take 6 x 32 cycles of the bf16 matrix cores against 8 x 64 of the
// float32 ones for the same 32 x 32 x 16 block.
//
// Tiles, waves, the split-K partials, the epilogue and the running sums are
// those of the float32 kernel (128 x 128 tiles, four 64 x 64 waves, a fold
// every kGemmSubK rows).  K advances in steps of XK = 16 rows: each thread
// loads two 16-byte chunks of each operand's step (rows t / 32 and t / 32 +
// 8, columns 4 (t % 32) ..) two steps ahead into registers, splits them
// and writes the three bf16 planes of the step into LDS ([k][m] rows, the
// 16-byte chunks swizzled as for the bf16 slabs); the waves then read
// their fragments with transposing reads.  Each value is split once per
// workgroup.  Planes are double buffered: the split of step s + 1 goes to
// the other buffer while the products of step s run, and one barrier per
// step separates them.
constexpr int XK = 16;                         // rows of K per step
constexpr int XPLANE = XK * BM;                // bf16 per plane of one operand (4 KB)
constexpr int XSUB = kGemmSubK / XK;           // steps per fold
typedef float xf4 __attribute__((ext_vector_type(4)));
typedef uint32_t xu2 __attribute__((ext_vector_type(2)));

// Buffer resource over rows [k0, min(k0 + XK, k_end)) of a float32 operand;
// rows past them read as zero, and the range ends at the operand's last
// element of the step's last row.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t step_rsrc(const void* base, int64_t ld, int k0, int k_end,
                                                            int cols) {
    const char* p = static_cast<const char*>(base) + (int64_t)k0 * ld * 4;
    const int rows = max(0, min(XK, k_end - k0));
    const int bytes = __builtin_amdgcn_readfirstlane(rows > 0 ? ((rows - 1) * (int)ld + cols) * 4 : 0);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0, bytes, 0x00020000);
}

// Splits four float32 values into three planes of four bf16 values (the
// low element of each pair in the low half).
__device__ __forceinline__ void split4(const xf4 v, xu2& p0, xu2& p1, xu2& p2) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float2v x = {v[2 * i], v[2 * i + 1]};
        const uint32_t u0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2v));
        const float2v x0 = {__builtin_bit_cast(float, u0 << 16), __builtin_bit_cast(float, u0 & 0xffff0000u)};
        const float2v r = {x[0] - x0[0], x[1] - x0[1]};
        const uint32_t u1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2v));
        const float2v r1 = {__builtin_bit_cast(float, u1 << 16), __builtin_bit_cast(float, u1 & 0xffff0000u)};
        const float2v r2 = {r[0] - r1[0], r[1] - r1[1]};
        p0[i] = u0;
        p1[i] = u1;
        p2[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r2, bf16x2v));
    }
}

// Transposing read at an immediate byte offset from `a`.
template <int OFF>
__device__ __forceinline__ short4v tr_read_at(uint32_t a) {
    short4v v;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(OFF));
    return v;
}

// Waits until at most N LDS reads are outstanding; the fragments of the
// reads it covers are named, so that no product that uses them moves above
// it (those of an edge wave's missing block are undefined and unread).
template <int N>
__device__ __forceinline__ void wait_frags(short4v (&f)[2][2]) {
    asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(f[0][0]), "+v"(f[0][1]), "+v"(f[1][0]), "+v"(f[1][1]) : "i"(N));
}

// The block products of one step for a wave: NA x NB of its 32 x 32 blocks
// (the others lie wholly past the problem's edge).  The step's planes lie
// at byte offset BASE of the plane buffers: A's plane q at BASE + q 4 KB,
// B's at BASE + BOFF + q 4 KB.  ra[a] / rb[b] hold this lane's address of
// its first read in A block a / B block b of plane 0; the other reads
// differ from it by immediates (the rows k0 + 4 + p / 4 lie 1 KB further).
// The reads run one plane ahead of the products: A0 meets B0, B1, B2 as
// they arrive, then A1 meets B0 and B1, and A2 (read into A0's registers)
// meets B0.  At most 12 reads are in flight, and the products go round the
// blocks so that none waits for the one before it on the same accumulator.
template <int NA, int NB, int BASE, int BOFF>
__device__ __forceinline__ void mma_x6(floatx16 (&acc)[2][2], const uint32_t (&ra)[2], const uint32_t (&rb)[2]) {
    constexpr int PL = XPLANE * 2;   // bytes per plane
    constexpr int RA = 2 * NA, RB = 2 * NB;   // reads per plane of A / B
    auto fr = [](const short4v& lo, const short4v& hi) {
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    short4v b0[2][2], b1[2][2], b2[2][2], a0[2][2], a1[2][2];
    auto rd = [&](short4v (&f)[2][2], const uint32_t (&r)[2], int n, auto off) {
        constexpr int OFF = decltype(off)::value;
#pragma unroll
        for (int q = 0; q < 2; ++q)
            if (q < n) {
                f[q][0] = tr_read_at<OFF>(r[q]);
                f[q][1] = tr_read_at<OFF + 1024>(r[q]);
            }
    };
    auto prod = [&](const short4v (&x)[2][2], const short4v (&y)[2][2]) {
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr(x[a][0], x[a][1]), fr(y[b][0], y[b][1]),
                                                                    acc[a][b], 0, 0, 0);
    };
    using std::integral_constant;
    rd(b0, rb, NB, integral_constant<int, BASE + BOFF>());
    rd(a0, ra, NA, integral_constant<int, BASE>());
    rd(b1, rb, NB, integral_constant<int, BASE + BOFF + PL>());
    wait_frags<RB>(b0);
    wait_frags<RB>(a0);
    prod(a0, b0);
    rd(b2, rb, NB, integral_constant<int, BASE + BOFF + 2 * PL>());
    wait_frags<RB>(b1);
    prod(a0, b1);
    rd(a1, ra, NA, integral_constant<int, BASE + PL>());
    wait_frags<RA>(b2);
    prod(a0, b2);
    rd(a0, ra, NA, integral_constant<int, BASE + 2 * PL>());   // A2
    wait_frags<RA>(a1);
    prod(a1, b0);
    prod(a1, b1);
    wait_frags<0>(a0);
    prod(a0, b0);
}

template <bool SAME>
__device__ __forceinline__ void gemm_x6_tile(const GemmLaunch& L, const TileWork& W, uint16_t* XS) {
    const GemmProb& P = W.P;
    const int k_begin = W.k_begin, k_end = W.k_end;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int wr = W.m0 + 64 * wm, wc = W.n0 + 64 * wn;
    const bool active = W.active && wr < P.M && wc < P.N;
    const bool a2 = wr + 32 < P.M, b2 = wc + 32 < P.N;
    // this thread's chunks: rows kt and kt + 8 of a step, columns mt .. mt + 3
    const int kt = tid >> 5, mt = 4 * (tid & 31);
    uint32_t offa[2], offb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        offa[j] = (W.m0 + mt < P.M) ? (uint32_t)(((kt + 8 * j) * P.lda + W.m0 + mt) * 4) : kOOB;
        offb[j] = (W.n0 + mt < P.N) ? (uint32_t)(((kt + 8 * j) * P.ldb + W.n0 + mt) * 4) : kOOB;
    }
    // this lane's first fragment read in each block (plane 0 of buffer 0)
    uint32_t ra[2], rb[2];
    {
        const int g = lane >> 4, p = lane & 15, k = 8 * (g >> 1) + (p >> 2);
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            ra[a] = lds_addr(XS + tr_at(k, wm * 64 + a * 32 + 16 * (g & 1) + 4 * (p & 3)));
            rb[a] = lds_addr(XS + tr_at(k, wn * 64 + a * 32 + 16 * (g & 1) + 4 * (p & 3)));
        }
    }
    // two steps of chunks in registers
    xf4 ra4[2][2], rb4[2][2];
    auto load = [&](int set, int k0) {
        const __amdgpu_buffer_rsrc_t rs = step_rsrc(P.a, P.lda, k0, k_end, P.M);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            ra4[set][j] = __builtin_bit_cast(xf4, __builtin_amdgcn_raw_buffer_load_b128(rs, offa[j], 0, 0));
        if (!SAME) {
            const __amdgpu_buffer_rsrc_t rt = step_rsrc(P.b, P.ldb, k0, k_end, P.N);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                rb4[set][j] = __builtin_bit_cast(xf4, __builtin_amdgcn_raw_buffer_load_b128(rt, offb[j], 0, 0));
        }
    };
    // splits register set `set` into the planes of buffer `buf`
    auto split = [&](int set, int buf) {
        uint16_t* const X = XS + buf * 6 * XPLANE;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int at = tr_at(kt + 8 * j, mt);
            xu2 p0, p1, p2;
            split4(ra4[set][j], p0, p1, p2);
            *reinterpret_cast<xu2*>(X + at) = p0;
            *reinterpret_cast<xu2*>(X + XPLANE + at) = p1;
            *reinterpret_cast<xu2*>(X + 2 * XPLANE + at) = p2;
            if (!SAME) {
                split4(rb4[set][j], p0, p1, p2);
                *reinterpret_cast<xu2*>(X + 3 * XPLANE + at) = p0;
                *reinterpret_cast<xu2*>(X + 4 * XPLANE + at) = p1;
                *reinterpret_cast<xu2*>(X + 5 * XPLANE + at) = p2;
            }
        }
    };
    constexpr int LPS = SAME ? 2 : 4;   // loads per step, per thread
    constexpr int BOFF = SAME ? 0 : 3 * XPLANE * 2;

    floatx16 acc[2][2], sum[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) { acc[a][b][r] = 0.0f; sum[a][b][r] = 0.0f; }
    const int nsteps = (k_end - k_begin + 2 * XK - 1) / (2 * XK) * 2;
    auto fold = [&]() {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                sum[a][b] += acc[a][b];
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
            }
    };
    // step s: planes in buffer s % 2, its chunks in register set s % 2.
    // Loads run two steps ahead and are issued for every step, also past
    // the end (their range is then empty and they read zeros without
    // touching memory): with no load left out on any path, the wait for
    // one register set leaves the other set's loads in flight.
    if (nsteps <= 0) {
        store_tile(P, L, sum, W.kc, W.t, W.m0, W.n0, wm, wn, lane);
        return;
    }
    load(0, k_begin);
    load(1, k_begin + XK);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS));
    split(0, 0);
    load(0, k_begin + 2 * XK);
    lds_barrier16();
    // The loop, compiled once per shape of the wave's work (NA x NB blocks;
    // none for a wave with nothing to compute), so that a step holds no
    // branch and the split of the next step can be scheduled among the
    // products of this one.  The step count is even (a last step past the
    // end reads zeros), and a fold every XSUB steps falls between pairs.
    auto run = [&](auto na, auto nb) {
        constexpr int NA = decltype(na)::value, NB = decltype(nb)::value;
        auto step = [&](int cur, auto h) {
            constexpr int H = decltype(h)::value;
            if constexpr (NA > 0) mma_x6<NA, NB, H * 6 * XPLANE * 2, BOFF>(acc, ra, rb);
            // step cur + 1's chunks (set 1 - H) have arrived once only step
            // cur + 2's (set H) are outstanding
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS));
            split(1 - H, 1 - H);
            load(1 - H, k_begin + (cur + 3) * XK);
            // the next step's planes are written and this step's are read
            lds_barrier16();
        };
        for (int st = 0; st < nsteps; st += 2) {
            step(st, std::integral_constant<int, 0>());
            step(st + 1, std::integral_constant<int, 1>());
            if constexpr (NA > 0)
                if ((st + 2) % XSUB == 0 || st + 2 == nsteps) fold();
        }
    };
    static_assert(XSUB % 2 == 0, "folds fall between pairs of steps");
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    if (!active) run(I0(), I0());
    else if (a2 && b2) run(I2(), I2());
    else if (a2) run(I2(), I1());
    else if (b2) run(I1(), I2());
    else run(I1(), I1());
    store_tile(P, L, sum, W.kc, W.t, W.m0, W.n0, wm, wn, lane);
}

__device__ __forceinline__ void gemm_x6_item(const GemmLaunch& L, int64_t items) {
    __shared__ __attribute__((aligned(16))) uint16_t XS[2 * 6 * XPLANE];
    const int64_t item = L.runs ? xcd_runs<kGemmRun>(blockIdx.x) : xcd_remap(blockIdx.x, gridDim.x);
    if (item >= items) return;
    const TileWork W = decode_item(L, item);
    if (W.same) gemm_x6_tile<true>(L, W, XS);
    else gemm_x6_tile<false>(L, W, XS);
}

__global__ __launch_bounds__(NT, 2) void factor_x6_kernel(GemmLaunch L, int64_t items) { gemm_x6_item(L, items); }
__global__ __launch_bounds__(NT, 2) void precond_x6_kernel(GemmLaunch L, int64_t items) { gemm_x6_item(L, items); }

// Sums the split-K partial tiles in chunk order and applies the epilogue.
// Each partial tile (T x T, T the launch's tile edge) is spread over
// T * T / 1024 workgroups; thread t sums four consecutive elements, with
// the loads of four chunks in flight.
__device__ __forceinline__ void gemm_reduce(const GemmLaunch& L, int64_t slices) {
    const int64_t g = blockIdx.x;
    if (g >= slices) return;
    const int T = L.tile;
    const int per_tile = T * T / (4 * NT);
    const int64_t tile = g / per_tile;
    const int slice = (int)(g % per_tile);
    const GemmProb P = L.probs[find_prob(L.probs, L.nprob, tile, true)];
    const int t = (int)(tile - P.red_begin);
    int ti, tj;
    tile_decode(P, t, ti, tj);
    const int e0 = slice * (4 * NT) + threadIdx.x * 4;
    const int64_t stride4 = (int64_t)P.ntiles * T * T / 4;
    const float4* base = reinterpret_cast<const float4*>(P.part + (int64_t)t * T * T + e0);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    int k = 0;
    for (; k + 4 <= P.ksplit; k += 4) {
        const float4 v0 = base[(k + 0) * stride4], v1 = base[(k + 1) * stride4];
        const float4 v2 = base[(k + 2) * stride4], v3 = base[(k + 3) * stride4];
        s.x += v0.x; s.y += v0.y; s.z += v0.z; s.w += v0.w;
        s.x += v1.x; s.y += v1.y; s.z += v1.z; s.w += v1.w;
        s.x += v2.x; s.y += v2.y; s.z += v2.z; s.w += v2.w;
        s.x += v3.x; s.y += v3.y; s.z += v3.z; s.w += v3.w;
    }
    for (; k < P.ksplit; ++k) {
        const float4 v = base[k * stride4];
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    const float sv[4] = {s.x, s.y, s.z, s.w};
    float res[4] = {0.f, 0.f, 0.f, 0.f};
    if (P.mode == kModeFactor && !L.first_step) {
#pragma unroll
        for (int q = 0; q < 4; ++q) res[q] = elem_prev(P, ti * T + (e0 + q) / T, tj * T + (e0 + q) % T);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) res[q] = elem_value(P, sv[q], res[q], L.eps, L.first_step);
#pragma unroll
    for (int q = 0; q < 4; ++q) elem_store(P, ti * T + (e0 + q) / T, tj * T + (e0 + q) % T, res[q]);
}

__global__ __launch_bounds__(NT) void factor_reduce_kernel(GemmLaunch L, int64_t slices) { gemm_reduce(L, slices); }
__global__ __launch_bounds__(NT) void precond_reduce_kernel(GemmLaunch L, int64_t slices) { gemm_reduce(L, slices); }

}  // namespace

hipError_t launch_gemm(const GemmLaunch& L, int64_t items, hipStream_t stream, bool bf16, bool factor,
                       bool bf16_aligned, bool bf16_edges) {
    if (items <= 0) return hipSuccess;
    // Items of different problems differ in cost (K chunks of different
    // length, diagonal tiles with an idle wave).  Large launches hand items to
    // the XCDs in runs, so that no XCD gets a range of only expensive ones;
    // small launches (fewer items than a few rounds of the chip) keep one
    // contiguous range per XCD.
    GemmLaunch R = L;
    R.runs = items >= kGemmRunsMin ? 1 : 0;
    const int64_t grid = R.runs ? (items + 8 * kGemmRun - 1) / (8 * kGemmRun) * (8 * kGemmRun) : items;
    if (bf16) {
        if (bf16_aligned && !bf16_edges)
            hipLaunchKernelGGL(factor_bf16_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, R, items);
        else if (bf16_aligned)
            hipLaunchKernelGGL(factor_bf16_edge_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, R, items);
        else
            hipLaunchKernelGGL(factor_bf16_any_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, R, items);
    } else if (factor) {
        hipLaunchKernelGGL(factor_x6_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, R, items);
    } else {
        hipLaunchKernelGGL(precond_x6_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, R, items);
    }
    return hipGetLastError();
}

hipError_t launch_factor_wide(const GemmLaunch& L, int64_t items, hipStream_t stream, bool edges) {
    if (items <= 0) return hipSuccess;
    GemmLaunch R = L;
    R.runs = items >= kGemmRunsMin ? 1 : 0;
    const int64_t grid = R.runs ? (items + 8 * kGemmRun - 1) / (8 * kGemmRun) * (8 * kGemmRun) : items;
    if (edges)
        hipLaunchKernelGGL(factor_bf16_wide_edge_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, R, items);
    else
        hipLaunchKernelGGL(factor_bf16_wide_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, R, items);
    return hipGetLastError();
}

hipError_t launch_gemm_reduce(const GemmLaunch& L, int64_t tiles, hipStream_t stream, bool factor) {
    if (tiles <= 0) return hipSuccess;
    const int64_t slices = tiles * (int64_t)(L.tile * L.tile / (4 * NT));
    if (factor)
        hipLaunchKernelGGL(factor_reduce_kernel, dim3((unsigned)slices), dim3(NT), 0, stream, L, slices);
    else
        hipLaunchKernelGGL(precond_reduce_kernel, dim3((unsigned)slices), dim3(NT), 0, stream, L, slices);
    return hipGetLastError();
}

}  // namespace kfac
