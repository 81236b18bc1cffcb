// Host side of the C ABI declared in include/kfac.h: argument validation,
// work planning, descriptor tables and launch sequences.  No device memory
// is allocated here; all scratch lives in the caller's workspace.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <numeric>
#include <vector>

#include "../../include/kfac.h"
#include "internal.h"

namespace kfac {
namespace {

__global__ void table_write_kernel(uint8_t* dst, TableChunk c, int nbytes) {
    for (int i = threadIdx.x; i < nbytes; i += blockDim.x) dst[i] = c.bytes[i];
}

constexpr size_t kAlign = 256;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Bump allocator over the caller's workspace (or a size-only dry run).
struct Carver {
    uint8_t* base;
    size_t used = 0;
    explicit Carver(void* b) : base(static_cast<uint8_t*>(b)) {}
    void* take(size_t bytes) {
        void* p = base ? base + used : nullptr;
        used = align_up(used + bytes, kAlign);
        return p;
    }
};

kfac_status_t hip_status(hipError_t e) { return e == hipSuccess ? KFAC_OK : KFAC_ERR_HIP; }

bool valid_dims(int n, const int64_t* d) {
    if (n < 1 || n > KFAC_MAX_COUNT || d == nullptr) return false;
    for (int i = 0; i < n; ++i)
        if (d[i] < 1 || d[i] > KFAC_MAX_DIM) return false;
    return true;
}

// ------------------------------------------------------------- factors --

struct FactorPlan {
    std::vector<GemmProb> probs;
    int64_t items = 0;
    int64_t red_tiles = 0;
    size_t part_bytes = 0;
    std::vector<int> repack;        // bf16 inputs of odd width, copied to an aligned pitch first
    size_t repack_bytes = 0;        // their copies, each 256-byte aligned
};

// Rows per K chunk: enough chunks overall to keep every CU busy, never so
// many that the partial tiles outweigh the work.  bf16 inputs of odd width
// are repacked to an aligned pitch first (bf16_repack.hip).
FactorPlan plan_factors(int n, const int64_t* rows, const int64_t* d, bool bf16) {
    FactorPlan p;
    p.probs.resize(n);
    double work = 0.0;
    for (int i = 0; i < n; ++i) {
        const int64_t t = ceil_div(d[i], kGemmTile);
        work += (double)(t * (t + 1) / 2) * (double)rows[i];
    }
    const double target_items = 8192.0;   // 16 per slot
    int64_t kc = (int64_t)std::ceil(work / target_items);
    kc = std::max<int64_t>(kc, 1024);
    kc = align_up(kc, kGemmSubK);
    int64_t part_elems = 0;
    for (int i = 0; i < n; ++i) {
        GemmProb& g = p.probs[i];
        std::memset(&g, 0, sizeof(g));
        const int64_t t = ceil_div(d[i], kGemmTile);
        g.lda = g.ldb = g.ldc = d[i];
        g.M = g.N = (int32_t)d[i];
        g.K = (int32_t)rows[i];
        g.tiles_m = g.tiles_n = (int32_t)t;
        g.ntiles = (int32_t)(t * (t + 1) / 2);
        const int64_t ksplit = std::max<int64_t>(1, ceil_div(rows[i], kc));
        g.ksplit = (int32_t)ksplit;
        g.kchunk = (int32_t)align_up(ceil_div(rows[i], ksplit), kGemmBK);
        g.mode = kModeFactor;
        g.alpha = (float)(1.0 / (double)rows[i]);
        g.item_begin = p.items;
        g.red_begin = p.red_tiles;
        p.items += (int64_t)g.ntiles * ksplit;
        if (ksplit > 1) {
            p.red_tiles += g.ntiles;
            part_elems += (int64_t)g.ntiles * ksplit * kGemmTile * kGemmTile;
        }
    }
    p.part_bytes = (size_t)part_elems * sizeof(float);
    for (int i = 0; bf16 && i < n; ++i) {
        if (d[i] % 2 == 0) continue;
        p.repack.push_back(i);
        p.repack_bytes += align_up((size_t)rows[i] * (size_t)repack_pitch(d[i]) * 2, kAlign);
    }
    return p;
}

// Workspace: the two tables next to each other (one upload), then the
// split-K partials and the repacked inputs.
size_t factors_ws(const FactorPlan& p, int n) {
    Carver c(nullptr);
    c.take(sizeof(GemmProb) * n);
    c.take(sizeof(RepackLayer) * p.repack.size());
    c.take(p.part_bytes);
    c.take(p.repack_bytes);
    return c.used;
}

// --------------------------------------------------------- precondition --

// Two launches of plain products per call: S^T = grad^T ginv, then
// P = (S^T)^T ainv.  When a launch has too few 128 x 128 tiles to give every
// CU several, K is split into equal chunks (partials summed in chunk order
// by the reduce kernel) so the last round of tiles is not left half empty;
// a cost estimate chooses between two split targets.
struct PrecondPlan {
    std::vector<GemmProb> p1, p2;
    int64_t items1 = 0, items2 = 0, red1 = 0, red2 = 0;
    size_t st_bytes = 0, part_bytes = 0;
};

constexpr int64_t kGemmSlots = 512;   // 256 CUs x 2 resident 128 x 128 tiles

// Chunk length for a split-K target of `per_slot` tiles per slot (0: no split).
int64_t plain_chunk(const std::vector<GemmProb>& probs, int per_slot) {
    int64_t tiles = 0;
    double work = 0.0;
    for (const GemmProb& g : probs) {
        tiles += g.ntiles;
        work += (double)g.ntiles * g.K;
    }
    if (tiles >= per_slot * kGemmSlots) return 0;
    return std::max<int64_t>(256, align_up((int64_t)std::ceil(work / ((double)per_slot * kGemmSlots)), 256));
}

// Estimated time of a launch in units of one 128 x 128 tile-row of products:
// the work spread over the slots, half the longest item for the last round,
// a fixed cost per item, and the split-K partials written and read back.
// Tiles with at most 32 valid rows or columns cost about a quarter.
double plain_cost(const std::vector<GemmProb>& probs, int64_t kc) {
    double total = 0.0, longest = 0.0, part_bytes = 0.0;
    for (const GemmProb& g : probs) {
        const int64_t ks = kc == 0 ? 1 : std::max<int64_t>(1, ceil_div(g.K, kc));
        const double rows = (double)align_up(ceil_div(g.K, ks), kGemmBK);
        int64_t thin = 0;
        if (g.M - (int64_t)kGemmTile * (g.tiles_m - 1) <= 32) thin += g.tiles_n;
        if (g.N - (int64_t)kGemmTile * (g.tiles_n - 1) <= 32) thin += g.tiles_m;
        thin = std::min<int64_t>(thin, g.ntiles);
        const double full = rows + 40.0, cheap = 0.25 * rows + 40.0;
        total += (double)ks * ((double)(g.ntiles - thin) * full + (double)thin * cheap);
        longest = std::max(longest, g.ntiles > thin ? full : cheap);
        if (ks > 1) part_bytes += 2.0 * (double)g.ntiles * ks * kGemmTile * kGemmTile * sizeof(float);
    }
    return total / kGemmSlots + 0.5 * longest + part_bytes / 6.4e5;
}

void plan_plain_launch(std::vector<GemmProb>& probs, int64_t& items, int64_t& red, int64_t& part_elems) {
    for (GemmProb& g : probs) {
        g.tiles_m = (int32_t)ceil_div(g.M, kGemmTile);
        g.tiles_n = (int32_t)ceil_div(g.N, kGemmTile);
        g.ntiles = g.tiles_m * g.tiles_n;
    }
    // split K for two or four tiles per slot (chunks of at least 256 rows),
    // whichever the cost estimate prefers
    const int64_t kc2 = plain_chunk(probs, 2), kc4 = plain_chunk(probs, 4);
    const int64_t kc = plain_cost(probs, kc2) < plain_cost(probs, kc4) ? kc2 : kc4;
    items = red = part_elems = 0;
    for (GemmProb& g : probs) {
        const int64_t ks = (kc == 0) ? 1 : std::max<int64_t>(1, ceil_div(g.K, kc));
        g.ksplit = (int32_t)ks;
        g.kchunk = (int32_t)align_up(ceil_div(g.K, ks), kGemmBK);
        g.mode = kModePlain;
        g.alpha = 1.0f;
        g.item_begin = items;
        g.red_begin = red;
        items += (int64_t)g.ntiles * ks;
        if (ks > 1) {
            red += g.ntiles;
            part_elems += (int64_t)g.ntiles * ks * kGemmTile * kGemmTile;
        }
    }
}

PrecondPlan plan_precondition(int n, const int64_t* d_g, const int64_t* d_a) {
    PrecondPlan p;
    p.p1.resize(n);
    p.p2.resize(n);
    for (int i = 0; i < n; ++i) {
        GemmProb& a = p.p1[i];
        std::memset(&a, 0, sizeof(a));
        a.lda = d_a[i];
        a.ldb = d_g[i];
        a.ldc = d_g[i];
        a.M = (int32_t)d_a[i];
        a.N = (int32_t)d_g[i];
        a.K = (int32_t)d_g[i];
        GemmProb& b = p.p2[i];
        std::memset(&b, 0, sizeof(b));
        b.lda = d_g[i];
        b.ldb = d_a[i];
        b.ldc = d_a[i];
        b.M = (int32_t)d_g[i];
        b.N = (int32_t)d_a[i];
        b.K = (int32_t)d_a[i];
        p.st_bytes += align_up(sizeof(float) * (size_t)(d_g[i] * d_a[i]), 256);
    }
    int64_t part1 = 0, part2 = 0;
    plan_plain_launch(p.p1, p.items1, p.red1, part1);
    plan_plain_launch(p.p2, p.items2, p.red2, part2);
    p.part_bytes = sizeof(float) * (size_t)std::max(part1, part2);   // the launches run one after the other
    return p;
}

size_t precondition_ws(int n, const int64_t* d_g, const int64_t* d_a) {
    const PrecondPlan p = plan_precondition(n, d_g, d_a);
    Carver c(nullptr);
    c.take(sizeof(GemmProb) * n);
    c.take(sizeof(GemmProb) * n);
    c.take(p.st_bytes);
    c.take(p.part_bytes);
    return c.used;
}

// -------------------------------------------------------------- inverse --

struct InvPlan {
    std::vector<int> order;  // matrices sorted by block count, largest first
    std::vector<InvBucket> buckets;
    int nbmax = 0;
};

InvPlan plan_inverse(int n, const int64_t* d) {
    InvPlan p;
    p.order.resize(n);
    std::iota(p.order.begin(), p.order.end(), 0);
    auto nb = [&](int i) { return (int)ceil_div(inv_extent(d[i]), kInvNB); };
    std::stable_sort(p.order.begin(), p.order.end(), [&](int a, int b) { return nb(a) > nb(b); });
    for (int s = 0; s < n; ++s) {
        const int b = nb(p.order[s]);
        if (p.buckets.empty() || p.buckets.back().nb != b) p.buckets.push_back(InvBucket{b, s, 0, 0});
        p.buckets.back().count++;
    }
    p.nbmax = nb(p.order[0]);
    return p;
}

// V = U^-1 is formed beside the potrf steps (two extra step launches at the
// end, no triangular-inverse launches) when those steps leave most of the
// chip idle: on average fewer than kFuseTilesPerStep trailing-update tiles
// per step (four per resident workgroup slot).  Otherwise the potrf steps
// are busy with the trailing update and V is formed afterwards by recursive
// doubling, in launches of its own.
constexpr int64_t kFuseTilesPerStep = 2048;
// Trailing updates of at least kPass2Tiles blocks run every second step
// (two panels deep) where V is formed beside potrf, every kDeepPass2-th step
// otherwise; of at least kPass3Tiles, every third or every kDeepPass3-th.
constexpr int64_t kPass2Tiles = 1024;
constexpr int64_t kPass3Tiles = 8192;
constexpr int kDeepPass2 = 4;
constexpr int kDeepPass3 = 8;
// Resident step-kernel workgroups (two per CU): the target count of row
// workgroups in a step without a trailing update.
constexpr int64_t kInvRowSlots = 512;
// Trailing updates of at least this many blocks (over several panels) get a
// launch of their own.
constexpr int64_t kApartTiles = 8192;

int64_t bucket_tiles(const InvPlan& p, int kind, int step, int rowq = 1);

bool fuse_v(const InvPlan& p) {
    int64_t tiles = 0;
    for (int k = 0; k < p.nbmax; ++k) tiles += bucket_tiles(p, kInvSyrk, k);
    return tiles < kFuseTilesPerStep * (int64_t)p.nbmax;
}

size_t inverse_ws(int n, const int64_t* d) {
    const bool fused = fuse_v(plan_inverse(n, d));
    Carver c(nullptr);
    c.take(sizeof(InvMat) * n);
    c.take(sizeof(InvBucket) * n);
    c.take(sizeof(GemmProb) * n);
    for (int i = 0; i < n; ++i) {
        const int64_t m = inv_extent(d[i]), nb = ceil_div(m, kInvNB), D = nb * kInvNB;
        c.take(sizeof(double) * (size_t)(D * D));
        c.take(sizeof(double) * (size_t)(D * kInvNB));
        if (fused) c.take(sizeof(double) * (size_t)(2 * vpart_slots(nb - 1) * kInvNB * kInvNB));
        if (m < d[i]) c.take(sizeof(double) * (size_t)border_doubles(nb));
        c.take(sizeof(float) * (size_t)((m + 1) * D));
    }
    return c.used;
}

int64_t bucket_tiles(const InvPlan& p, int kind, int step, int rowq) {
    int64_t t = 0;
    for (const InvBucket& b : p.buckets) t += inv_tiles(kind, b.nb, step, rowq) * b.count;
    return t;
}

// -------------------------------------------------------------- packing --

size_t pack_ws(int n) {
    Carver c(nullptr);
    c.take(sizeof(PackSrc) * n);
    c.take(sizeof(PackLayer) * n);
    return c.used;
}

}  // namespace

hipError_t upload_table(void* dst_device, const void* src_host, size_t nbytes, hipStream_t stream) {
    const uint8_t* src = static_cast<const uint8_t*>(src_host);
    uint8_t* dst = static_cast<uint8_t*>(dst_device);
    for (size_t off = 0; off < nbytes; off += kTableChunk) {
        TableChunk c;
        const size_t nb = std::min<size_t>(kTableChunk, nbytes - off);
        std::memcpy(c.bytes, src + off, nb);
        hipLaunchKernelGGL(table_write_kernel, dim3(1), dim3(256), 0, stream, dst + off, c, (int)nb);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Several tables carved one after another from the workspace, uploaded as
// one stretch (the alignment gaps between them written as zeros), so that
// they cost the launches of one table.
struct TablePart {
    void* dst;
    const void* src;
    size_t bytes;
};
hipError_t upload_tables(std::initializer_list<TablePart> parts, hipStream_t stream) {
    uint8_t* lo = static_cast<uint8_t*>(parts.begin()->dst);
    uint8_t* hi = lo;
    for (const TablePart& t : parts) {
        uint8_t* d = static_cast<uint8_t*>(t.dst);
        if (d < lo) return hipErrorInvalidValue;
        hi = std::max(hi, d + t.bytes);
    }
    std::vector<uint8_t> blob((size_t)(hi - lo), 0);
    for (const TablePart& t : parts) std::memcpy(blob.data() + (static_cast<uint8_t*>(t.dst) - lo), t.src, t.bytes);
    return upload_table(lo, blob.data(), blob.size(), stream);
}

namespace {

// --------------------------------------------------------------- packing --

kfac_status_t pack_args(int n, float* const* m, const int64_t* d, const float* packed, kfac_pack_dir_t dir) {
    if (!valid_dims(n, d) || m == nullptr || packed == nullptr || !aligned(packed, 4)) return KFAC_ERR_INVALID_VALUE;
    if (dir != KFAC_PACK && dir != KFAC_UNPACK) return KFAC_ERR_INVALID_VALUE;
    for (int i = 0; i < n; ++i)
        if (m[i] == nullptr || !aligned(m[i], 4)) return KFAC_ERR_INVALID_VALUE;
    return KFAC_OK;
}

// The host keeps only the totals that size the grid; the per-layer offsets
// are prefix sums formed on the device, in the tables carved from `ws`.
hipError_t pack_run(int n, float* const* m, const int64_t* d, float* packed, kfac_pack_dir_t dir, void* ws,
                    hipStream_t stream) {
    std::vector<PackSrc> src(n);
    int64_t total = 0, tiles = 0;
    for (int i = 0; i < n; ++i) {
        src[i] = PackSrc{m[i], d[i]};
        const int64_t t1 = ceil_div(d[i], kUnpackTile);
        total += d[i] * (d[i] + 1) / 2;
        tiles += t1 * (t1 + 1) / 2;
    }
    Carver c(ws);
    PackSrc* src_dev = static_cast<PackSrc*>(c.take(sizeof(PackSrc) * n));
    PackLayer* layers_dev = static_cast<PackLayer*>(c.take(sizeof(PackLayer) * n));
    hipError_t e = upload_table(src_dev, src.data(), sizeof(PackSrc) * n, stream);
    if (e == hipSuccess) e = launch_pack_table(src_dev, n, layers_dev, stream);
    if (e == hipSuccess)
        e = dir == KFAC_PACK ? launch_pack(layers_dev, n, packed, total, stream)
                             : launch_unpack(layers_dev, n, packed, tiles, stream);
    return e;
}

// ------------------------------------------------- allocation-free scratch --
// The tables of kfac_pack_sym_static live in this array instead of a
// caller's workspace.  In host code `scratch` names a host-side stand-in,
// not the device memory: its device address is looked up once per device
// (with that device current) and only that address is handed to kernels.
constexpr size_t kStaticScratchBytes = 64 * 1024;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t static_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

}  // namespace kfac

using namespace kfac;

extern "C" {

int kfac_abi_version(void) { return 1; }

const char* kfac_status_string(kfac_status_t s) {
    switch (s) {
        case KFAC_OK: return "KFAC_OK";
        case KFAC_ERR_INVALID_VALUE: return "KFAC_ERR_INVALID_VALUE";
        case KFAC_ERR_WORKSPACE: return "KFAC_ERR_WORKSPACE";
        case KFAC_ERR_UNSUPPORTED: return "KFAC_ERR_UNSUPPORTED";
        case KFAC_ERR_HIP: return "KFAC_ERR_HIP";
    }
    return "KFAC_ERR_UNKNOWN";
}

// ---------------------------------------------------------------- factors --

size_t kfac_factors_workspace_size(int n, const int64_t* rows, const int64_t* d, kfac_dtype_t in_dtype) {
    if (!valid_dims(n, d) || rows == nullptr || (in_dtype != KFAC_F32 && in_dtype != KFAC_BF16)) return 0;
    for (int i = 0; i < n; ++i)
        if (rows[i] < 1 || rows[i] > INT32_MAX) return 0;
    return factors_ws(plan_factors(n, rows, d, in_dtype == KFAC_BF16), n);
}

kfac_status_t kfac_factors(int n, const void* const* x, const int64_t* rows, const int64_t* d,
                           kfac_dtype_t in_dtype, float* const* m, float eps, int first_step,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!valid_dims(n, d) || x == nullptr || rows == nullptr || m == nullptr) return KFAC_ERR_INVALID_VALUE;
    if (in_dtype != KFAC_F32 && in_dtype != KFAC_BF16) return KFAC_ERR_INVALID_VALUE;
    if (!std::isfinite(eps) || eps < 0.0f || eps > 1.0f) return KFAC_ERR_INVALID_VALUE;
    const size_t esz = in_dtype == KFAC_BF16 ? 2 : 4;
    for (int i = 0; i < n; ++i) {
        if (rows[i] < 1 || rows[i] > INT32_MAX) return KFAC_ERR_INVALID_VALUE;
        if (x[i] == nullptr || m[i] == nullptr || !aligned(x[i], esz) || !aligned(m[i], 4)) return KFAC_ERR_INVALID_VALUE;
    }
    const bool bf16 = in_dtype == KFAC_BF16;
    FactorPlan p = plan_factors(n, rows, d, bf16);
    const size_t need = factors_ws(p, n);
    if (workspace == nullptr || !aligned(workspace, kAlign) || workspace_bytes < need) return KFAC_ERR_WORKSPACE;

    Carver c(workspace);
    GemmProb* probs_dev = static_cast<GemmProb*>(c.take(sizeof(GemmProb) * n));
    RepackLayer* repack_dev = static_cast<RepackLayer*>(c.take(sizeof(RepackLayer) * p.repack.size()));
    float* part = static_cast<float*>(c.take(p.part_bytes));
    uint8_t* repack_buf = static_cast<uint8_t*>(c.take(p.repack_bytes));
    std::vector<RepackLayer> rl(p.repack.size());
    int64_t repack_blocks = 0;
    for (size_t r = 0; r < p.repack.size(); ++r) {
        const int i = p.repack[r];
        const int64_t pitch = repack_pitch(d[i]);
        rl[r] = RepackLayer{static_cast<const uint16_t*>(x[i]), reinterpret_cast<uint16_t*>(repack_buf), rows[i],
                            repack_blocks, (int32_t)d[i], (int32_t)pitch};
        repack_buf += align_up((size_t)rows[i] * (size_t)pitch * 2, kAlign);
        repack_blocks += ceil_div(rows[i] * (pitch / 8), 256);
    }
    int64_t part_off = 0;
    for (size_t r = 0; r < p.repack.size(); ++r) {
        GemmProb& g = p.probs[p.repack[r]];
        g.a = g.b = rl[r].dst;
        g.lda = g.ldb = rl[r].pitch;
    }
    for (int i = 0; i < n; ++i) {
        GemmProb& g = p.probs[i];
        if (g.a == nullptr) g.a = g.b = x[i];
        g.c = m[i];
        g.bf16 = bf16;
        if (g.ksplit > 1) {
            g.part = part + part_off;
            part_off += (int64_t)g.ntiles * g.ksplit * kGemmTile * kGemmTile;
        }
    }
    // bf16 rows that all start 4-byte aligned (every input after the repack,
    // unless a base is one element off) take the kernels without the
    // element-wise path; with no split of K, at most kWideMaxK rows and
    // enough tiles, the wide tiles
    bool aligned_rows = true, edges = false, wide = bf16, wide_edges = false;
    int64_t wide_items = 0;
    for (int i = 0; i < n; ++i) {
        const GemmProb& g = p.probs[i];
        aligned_rows = aligned_rows && (g.lda & 1) == 0 && aligned(g.a, 4);
        edges = edges || g.M % kGemmTile != 0;
        wide = wide && g.ksplit == 1 && g.K <= kWideMaxK;
        wide_edges = wide_edges || g.M % kWideM != 0;
        wide_items += wide_tiles(g.M);
    }
    wide = wide && aligned_rows && wide_items >= kWideMinTiles;
    if (wide) {
        int64_t item = 0;
        for (int i = 0; i < n; ++i) {
            GemmProb& g = p.probs[i];
            g.tiles_m = (int32_t)ceil_div((int64_t)g.M, (int64_t)kWideM);
            g.tiles_n = (int32_t)ceil_div((int64_t)g.N, (int64_t)kWideN);
            g.ntiles = (int32_t)wide_tiles(g.M);
            g.item_begin = item;
            item += g.ntiles;
        }
    }
    hipError_t e = rl.empty() ? upload_table(probs_dev, p.probs.data(), sizeof(GemmProb) * n, stream)
                              : upload_tables({{probs_dev, p.probs.data(), sizeof(GemmProb) * n},
                                               {repack_dev, rl.data(), sizeof(RepackLayer) * rl.size()}},
                                              stream);
    if (e == hipSuccess && !rl.empty()) e = launch_repack_bf16(repack_dev, (int)rl.size(), repack_blocks, stream);
    if (e != hipSuccess) return KFAC_ERR_HIP;
    GemmLaunch L{probs_dev, n, first_step ? 1 : 0, eps, 0, kGemmTile};
    if (wide) return hip_status(launch_factor_wide(L, wide_items, stream, wide_edges));
    e = launch_gemm(L, p.items, stream, bf16, true, aligned_rows, edges);
    if (e != hipSuccess) return KFAC_ERR_HIP;
    return hip_status(launch_gemm_reduce(L, p.red_tiles, stream, true));
}

// ------------------------------------------------------------------- pack --

int64_t kfac_packed_size(int n, const int64_t* d) {
    if (!valid_dims(n, d)) return -1;
    int64_t s = 0;
    for (int i = 0; i < n; ++i) s += d[i] * (d[i] + 1) / 2;
    return s;
}

size_t kfac_pack_workspace_size(int n, const int64_t* d) {
    if (!valid_dims(n, d)) return 0;
    return pack_ws(n);
}

kfac_status_t kfac_pack_sym(int n, float* const* m, const int64_t* d, float* packed, kfac_pack_dir_t dir,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const kfac_status_t st = pack_args(n, m, d, packed, dir);
    if (st != KFAC_OK) return st;
    const size_t need = pack_ws(n);
    if (workspace == nullptr || !aligned(workspace, kAlign) || workspace_bytes < need) return KFAC_ERR_WORKSPACE;
    return hip_status(pack_run(n, m, d, packed, dir, workspace, stream));
}

kfac_status_t kfac_pack_sym_static(int n, float* const* m, const int64_t* d, float* packed, kfac_pack_dir_t dir,
                                   hipStream_t stream) {
    const kfac_status_t st = pack_args(n, m, d, packed, dir);
    if (st != KFAC_OK) return st;
    if (n > KFAC_STATIC_MAX_FACTORS) return KFAC_ERR_UNSUPPORTED;
    static_assert(kStaticScratchBytes >= (sizeof(PackSrc) + sizeof(PackLayer)) * KFAC_STATIC_MAX_FACTORS + 2 * kAlign,
                  "the static scratch holds the tables of KFAC_STATIC_MAX_FACTORS factors");
    void* ws = nullptr;
    hipError_t e = static_scratch(&ws);
    if (e == hipSuccess) e = pack_run(n, m, d, packed, dir, ws, stream);
    return hip_status(e);
}

kfac_status_t kfac_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
    if (bytes % 16 != 0) return KFAC_ERR_INVALID_VALUE;
    if (bytes == 0) return KFAC_OK;
    if (src == nullptr || dst == nullptr || !aligned(src, 16) || !aligned(dst, 16)) return KFAC_ERR_INVALID_VALUE;
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    if (a < b + bytes && b < a + bytes) return KFAC_ERR_INVALID_VALUE;
    return hip_status(launch_stream_copy(src, dst, bytes, stream));
}

// ---------------------------------------------------------------- inverse --

size_t kfac_inverse_workspace_size(int n, const int64_t* d) {
    if (!valid_dims(n, d)) return 0;
    return inverse_ws(n, d);
}

kfac_status_t kfac_damped_inverse(int n, const float* const* x, const int64_t* d, float gamma,
                                  float* const* xinv, int32_t* info,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!valid_dims(n, d) || x == nullptr || xinv == nullptr || info == nullptr || !aligned(info, 4))
        return KFAC_ERR_INVALID_VALUE;
    if (!std::isfinite(gamma) || gamma < 0.0f) return KFAC_ERR_INVALID_VALUE;
    for (int i = 0; i < n; ++i)
        if (x[i] == nullptr || xinv[i] == nullptr || !aligned(x[i], 4) || !aligned(xinv[i], 4))
            return KFAC_ERR_INVALID_VALUE;
    const size_t need = inverse_ws(n, d);
    if (workspace == nullptr || !aligned(workspace, kAlign) || workspace_bytes < need) return KFAC_ERR_WORKSPACE;

    InvPlan p = plan_inverse(n, d);
    const bool fused = fuse_v(p);
    Carver c(workspace);
    InvMat* mats_dev = static_cast<InvMat*>(c.take(sizeof(InvMat) * n));
    InvBucket* buckets_dev = static_cast<InvBucket*>(c.take(sizeof(InvBucket) * n));
    GemmProb* gprobs_dev = static_cast<GemmProb*>(c.take(sizeof(GemmProb) * n));
    // per-matrix scratch in original order
    std::vector<double*> w(n), dinv(n), part(n), bvec(n);
    std::vector<float*> vt(n);
    bool bordered = false;
    for (int i = 0; i < n; ++i) {
        const int64_t m = inv_extent(d[i]), nb = ceil_div(m, kInvNB), D = nb * kInvNB;
        w[i] = static_cast<double*>(c.take(sizeof(double) * (size_t)(D * D)));
        dinv[i] = static_cast<double*>(c.take(sizeof(double) * (size_t)(D * kInvNB)));
        part[i] = fused ? static_cast<double*>(c.take(sizeof(double) * (size_t)(2 * vpart_slots(nb - 1) * kInvNB * kInvNB)))
                          : nullptr;
        bvec[i] = m < d[i] ? static_cast<double*>(c.take(sizeof(double) * (size_t)border_doubles(nb))) : nullptr;
        vt[i] = static_cast<float*>(c.take(sizeof(float) * (size_t)((m + 1) * D)));
        bordered = bordered || m < d[i];
    }
    std::vector<InvMat> mats(n);
    for (int s = 0; s < n; ++s) {
        const int i = p.order[s];
        const int64_t m = inv_extent(d[i]);
        mats[s] = InvMat{x[i], xinv[i], w[i], dinv[i], info + i, part[i], bvec[i], vt[i], (int32_t)d[i], (int32_t)m,
                         (int32_t)ceil_div(m, kInvNB), 0};
    }
    // The last product Z = V V^T (plus v v^T for a bordered matrix) on the
    // GEMM of the factor stage: Aop = Bop = V^T in float32 (row k holds
    // V_ik, zero for k < i), upper tiles with K from max(row, column), both
    // triangles written.  Matrices in the bucket order (largest first).
    std::vector<GemmProb> gp(n);
    int64_t gitems = 0;
    for (int s = 0; s < n; ++s) {
        const int i = p.order[s];
        const int64_t m = inv_extent(d[i]), D = ceil_div(m, kInvNB) * kInvNB, t = ceil_div(m, kGemmTile);
        GemmProb& g = gp[s];
        std::memset(&g, 0, sizeof(g));
        g.a = g.b = vt[i];
        g.c = xinv[i];
        g.lda = g.ldb = D;
        g.ldc = d[i];
        g.M = g.N = (int32_t)m;
        g.K = (int32_t)(m + (m < d[i] ? 1 : 0));
        g.tiles_m = g.tiles_n = (int32_t)t;
        g.ntiles = (int32_t)(t * (t + 1) / 2);
        g.ksplit = 1;
        g.kchunk = (int32_t)align_up(g.K, kGemmBK);
        g.mode = kModeFactor;
        g.alpha = 1.0f;
        g.flags = kGemmTriK | kGemmMirror;
        g.item_begin = gitems;
        gitems += g.ntiles;
    }
    hipError_t e = upload_tables({{mats_dev, mats.data(), sizeof(InvMat) * n},
                                  {buckets_dev, p.buckets.data(), sizeof(InvBucket) * p.buckets.size()},
                                  {gprobs_dev, gp.data(), sizeof(GemmProb) * n}},
                                 stream);
    if (e != hipSuccess) return KFAC_ERR_HIP;

    InvLaunch L{mats_dev, buckets_dev, (int32_t)p.buckets.size(), 0, (double)gamma, 0, 0, 0, 0, fused ? 1 : 0, 0, 1, 0, 0};
    bool next_done = false;   // the step before updated this step's row with its pending panels
    int last_pass = 0;   // rows below the last trailing update hold the updates of panels [0, last_pass)
    e = launch_inv_prepare(L, bucket_tiles(p, kInvPrepare, 0), stream);
    // with V formed beside potrf, two more launches finish its last columns
    const int nsteps = fused ? p.nbmax + 2 : p.nbmax;
    for (int k = 0; e == hipSuccess && k < nsteps; ++k) {
        // row-k blocks of every matrix in the first workgroups (spread over the
        // XCDs as dispatched), then the columns of V, then the trailing update
        // from a multiple of 8
        L.step = k;
        L.plo = last_pass;
        L.rplo = next_done ? k - 1 : last_pass;
        // A heavy trailing update (it rewrites its blocks in full) runs only
        // every few steps, that many panels deep; the rows in between take the
        // skipped panels from the next-row workgroups of the step before
        // (below), and apply only the last panel themselves.  Where V is
        // formed beside potrf there are no next-row workgroups, the rows
        // apply every skipped panel, and the depth stays within
        // kMaxPassDepth.  A step with no trailing blocks at all (no rows below
        // it) counts as an update.
        int64_t trail = bucket_tiles(p, kInvSyrk, k);
        const int depth = fused ? (trail >= kPass3Tiles ? 3 : trail >= kPass2Tiles ? 2 : 1)
                                : (trail >= kPass3Tiles ? kDeepPass3 : trail >= kPass2Tiles ? kDeepPass2 : 1);
        static_assert(kMaxPassDepth >= 3, "three-panel updates where the rows apply every skipped panel");
        if (k - last_pass >= depth || trail == 0) last_pass = k;
        else trail = 0;
        // Every row workgroup factors the diagonal block itself.  In a step
        // without a trailing update, more row blocks than resident slots
        // would take several rounds of that factorisation; there each
        // workgroup takes rowq consecutive blocks of the row instead, so
        // that one round holds them all.
        const int64_t rows1 = bucket_tiles(p, kInvPanel, k);
        L.rowq = trail == 0 && !fused ? (int32_t)std::max<int64_t>(1, ceil_div(rows1, kInvRowSlots)) : 1;
        L.split = bucket_tiles(p, kInvPanel, k, L.rowq);
        L.fin_end = L.split + (fused ? bucket_tiles(p, kInvVFin, k) : 0);
        L.part_end = L.fin_end + (fused ? bucket_tiles(p, kInvVPart, k) : 0);
        // In a step without a trailing update, row k + 1 takes the panels
        // [plo, k) that it lacks in this launch, beside (after) the row
        // workgroups, instead of on the chain of the next step.  (Not where
        // V is formed beside potrf: there the step launches are short and
        // the extra workgroups cost more than they take off the chain.)
        next_done = !fused && trail == 0 && k > L.plo && k + 1 < p.nbmax;
        L.next_end = L.part_end + (next_done ? bucket_tiles(p, kInvNextRow, k) : 0);
        // Large multi-panel trailing updates run as a launch of their own, at
        // four workgroups per CU (the step kernel holds two), before the
        // step's launch; smaller ones stay in it, beside its row workgroups,
        // whose chain would otherwise stand alone.  The two touch disjoint
        // blocks: rows below k, against row k and the panels above it.
        const bool apart = trail >= kApartTiles && k - L.plo > 1;
        if (apart) {
            e = launch_inv_trail(L, trail, stream);
            trail = 0;
        }
        L.tail_first = trail > 0 ? (L.next_end + 7) / 8 * 8 : L.next_end;
        if (e == hipSuccess && L.tail_first + trail > 0) e = launch_inv_step(L, L.tail_first + trail, stream);
    }
    for (int lvl = 0; !fused && e == hipSuccess && (1 << lvl) < p.nbmax; ++lvl) {   // bottom level first
        L.step = lvl;
        const int64_t t = bucket_tiles(p, kInvTrtri, lvl);
        e = launch_inv_trtri_a(L, t, stream);
        if (e == hipSuccess) e = launch_inv_trtri_b(L, t, stream);
    }
    if (bordered && e == hipSuccess) {
        // the last row and column of the bordered matrices: w = V^T x, u = V w,
        // then mu^2 = xi - w^T w, v = -u / mu and the border of the output
        L.step = 0;
        const int64_t runs = bucket_tiles(p, kInvBorderRun, 0);
        e = launch_inv_border_w(L, runs, stream);
        if (e == hipSuccess) e = launch_inv_border_u(L, runs, stream);
        if (e == hipSuccess) e = launch_inv_border_v(L, bucket_tiles(p, kInvBorder, 0), stream);
    }
    if (e == hipSuccess) {
        L.step = 0;
        e = launch_inv_vt32(L, bucket_tiles(p, kInvUpper, 0), stream);
    }
    if (e == hipSuccess) {
        const GemmLaunch G{gprobs_dev, n, 1, 1.0f, 0, kGemmTile};
        e = launch_gemm(G, gitems, stream, false, true);
    }
    return hip_status(e);
}

// ----------------------------------------------------------- precondition --

size_t kfac_precondition_workspace_size(int n, const int64_t* d_g, const int64_t* d_a) {
    if (!valid_dims(n, d_g) || !valid_dims(n, d_a)) return 0;
    return precondition_ws(n, d_g, d_a);
}

kfac_status_t kfac_precondition(int n, const float* const* ginv, const float* const* grad,
                                const float* const* ainv, const int64_t* d_g, const int64_t* d_a,
                                float* const* out, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
    if (!valid_dims(n, d_g) || !valid_dims(n, d_a) || ginv == nullptr || grad == nullptr || ainv == nullptr ||
        out == nullptr)
        return KFAC_ERR_INVALID_VALUE;
    for (int i = 0; i < n; ++i) {
        if (ginv[i] == nullptr || grad[i] == nullptr || ainv[i] == nullptr || out[i] == nullptr)
            return KFAC_ERR_INVALID_VALUE;
        if (!aligned(ginv[i], 4) || !aligned(grad[i], 4) || !aligned(ainv[i], 4) || !aligned(out[i], 4))
            return KFAC_ERR_INVALID_VALUE;
    }
    const size_t need = precondition_ws(n, d_g, d_a);
    if (workspace == nullptr || !aligned(workspace, kAlign) || workspace_bytes < need) return KFAC_ERR_WORKSPACE;

    PrecondPlan p = plan_precondition(n, d_g, d_a);
    Carver c(workspace);
    GemmProb* p1_dev = static_cast<GemmProb*>(c.take(sizeof(GemmProb) * n));
    GemmProb* p2_dev = static_cast<GemmProb*>(c.take(sizeof(GemmProb) * n));
    float* st_base = static_cast<float*>(c.take(p.st_bytes));
    float* part = static_cast<float*>(c.take(p.part_bytes));
    size_t st_off = 0;
    int64_t part1 = 0, part2 = 0;
    for (int i = 0; i < n; ++i) {
        float* st = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(st_base) + st_off);
        st_off += align_up(sizeof(float) * (size_t)(d_g[i] * d_a[i]), 256);
        GemmProb& a = p.p1[i];   // S^T [d_a][d_g] = grad^T . ginv   (ginv symmetric)
        a.a = grad[i];
        a.b = ginv[i];
        a.c = st;
        GemmProb& b = p.p2[i];   // P [d_g][d_a] = (S^T)^T . ainv
        b.a = st;
        b.b = ainv[i];
        b.c = out[i];
        if (a.ksplit > 1) {
            a.part = part + part1;
            part1 += (int64_t)a.ntiles * a.ksplit * kGemmTile * kGemmTile;
        }
        if (b.ksplit > 1) {
            b.part = part + part2;
            part2 += (int64_t)b.ntiles * b.ksplit * kGemmTile * kGemmTile;
        }
    }
    hipError_t e = upload_tables({{p1_dev, p.p1.data(), sizeof(GemmProb) * n}, {p2_dev, p.p2.data(), sizeof(GemmProb) * n}},
                                 stream);
    if (e != hipSuccess) return KFAC_ERR_HIP;
    GemmLaunch L1{p1_dev, n, 0, 0.0f, 0, kGemmTile};
    e = launch_gemm(L1, p.items1, stream, false, false);
    if (e == hipSuccess) e = launch_gemm_reduce(L1, p.red1, stream, false);
    if (e != hipSuccess) return KFAC_ERR_HIP;
    GemmLaunch L2{p2_dev, n, 0, 0.0f, 0, kGemmTile};
    e = launch_gemm(L2, p.items2, stream, false, false);
    if (e == hipSuccess) e = launch_gemm_reduce(L2, p.red2, stream, false);
    return hip_status(e);
}

// ----------------------------------------------------------------- layers --

size_t kfac_im2col_workspace_size(int n) {
    if (n < 1 || n > KFAC_MAX_COUNT) return 0;
    Carver c(nullptr);
    c.take(sizeof(Im2colLayer) * n);
    return c.used;
}

kfac_status_t kfac_im2col(int n, const void* const* x, const kfac_conv_t* shape, kfac_dtype_t dtype,
                          void* const* a, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (n < 1 || n > KFAC_MAX_COUNT || x == nullptr || shape == nullptr || a == nullptr) return KFAC_ERR_INVALID_VALUE;
    if (dtype != KFAC_F32 && dtype != KFAC_BF16) return KFAC_ERR_INVALID_VALUE;
    const size_t esz = dtype == KFAC_BF16 ? 2 : 4;
    std::vector<Im2colLayer> layers(n);
    int64_t tiles = 0;
    for (int i = 0; i < n; ++i) {
        const kfac_conv_t& s = shape[i];
        if (x[i] == nullptr || a[i] == nullptr || !aligned(x[i], esz) || !aligned(a[i], esz)) return KFAC_ERR_INVALID_VALUE;
        if (s.n < 1 || s.c < 1 || s.h < 1 || s.w < 1 || s.kh < 1 || s.kw < 1 || s.sh < 1 || s.sw < 1 || s.ph < 0 ||
            s.pw < 0 || s.dh < 1 || s.dw < 1 || (s.ones != 0 && s.ones != 1) || s.reserved != 0)
            return KFAC_ERR_INVALID_VALUE;
        const int64_t eh = s.h + 2 * (int64_t)s.ph - (int64_t)s.dh * (s.kh - 1) - 1;
        const int64_t ew = s.w + 2 * (int64_t)s.pw - (int64_t)s.dw * (s.kw - 1) - 1;
        if (eh < 0 || ew < 0) return KFAC_ERR_INVALID_VALUE;
        const int64_t oh = eh / s.sh + 1, ow = ew / s.sw + 1;
        const int64_t cols = s.c * s.kh * s.kw + s.ones;
        const int64_t rows = s.n * oh * ow;
        if (oh > INT32_MAX || ow > INT32_MAX || cols > INT32_MAX || rows > INT32_MAX / cols ||
            s.c > INT32_MAX / s.h / s.w)
            return KFAC_ERR_INVALID_VALUE;
        Im2colLayer& L = layers[i];
        L = Im2colLayer{x[i], a[i], s.c, s.h, s.w, rows, tiles, s.kh, s.kw, s.sh, s.sw, s.ph, s.pw, s.dh, s.dw,
                        (int32_t)oh, (int32_t)ow, (int32_t)cols, s.ones, (int32_t)ceil_div(cols, kLayerTile), 0};
        if (s.kh == 1 && s.kw == 1 && s.sh == 1 && s.sw == 1 && s.ph == 0 && s.pw == 0 && (s.h * s.w) % 4 == 0 &&
            aligned(x[i], 4 * esz))
            L.vec |= kVecIn;
        if (cols % 4 == 0 && aligned(a[i], 4 * esz)) L.vec |= kVecOut;
        tiles += ceil_div(rows, kLayerTile) * L.tiles_c;
    }
    const size_t need = kfac_im2col_workspace_size(n);
    if (workspace == nullptr || !aligned(workspace, kAlign) || workspace_bytes < need) return KFAC_ERR_WORKSPACE;
    Carver c(workspace);
    Im2colLayer* dev = static_cast<Im2colLayer*>(c.take(sizeof(Im2colLayer) * n));
    hipError_t e = upload_table(dev, layers.data(), sizeof(Im2colLayer) * n, stream);
    if (e != hipSuccess) return KFAC_ERR_HIP;
    return hip_status(launch_im2col(dev, n, tiles, dtype == KFAC_BF16, stream));
}

size_t kfac_grad_rows_workspace_size(int n) {
    if (n < 1 || n > KFAC_MAX_COUNT) return 0;
    Carver c(nullptr);
    c.take(sizeof(GradRowsLayer) * n);
    return c.used;
}

kfac_status_t kfac_grad_rows(int n, const void* const* gy, const int64_t* batch, const int64_t* ch,
                             const int64_t* hw, kfac_dtype_t dtype, float scale, void* const* g,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (n < 1 || n > KFAC_MAX_COUNT || gy == nullptr || batch == nullptr || ch == nullptr || hw == nullptr ||
        g == nullptr || !std::isfinite(scale))
        return KFAC_ERR_INVALID_VALUE;
    if (dtype != KFAC_F32 && dtype != KFAC_BF16) return KFAC_ERR_INVALID_VALUE;
    const size_t esz = dtype == KFAC_BF16 ? 2 : 4;
    std::vector<GradRowsLayer> layers(n);
    int64_t tiles = 0;
    for (int i = 0; i < n; ++i) {
        if (gy[i] == nullptr || g[i] == nullptr || !aligned(gy[i], esz) || !aligned(g[i], esz)) return KFAC_ERR_INVALID_VALUE;
        if (batch[i] < 1 || ch[i] < 1 || hw[i] < 1) return KFAC_ERR_INVALID_VALUE;
        const int64_t tc = ceil_div(ch[i], kLayerTile);
        const int64_t tp = hw[i] == 1 ? ceil_div(batch[i], kLayerTile) : ceil_div(hw[i], kLayerTile);
        if (tc > INT32_MAX || tp > INT32_MAX) return KFAC_ERR_INVALID_VALUE;
        layers[i] = GradRowsLayer{gy[i], g[i], batch[i], ch[i], hw[i], tiles, (int32_t)tc, (int32_t)tp, 0, 0};
        if (hw[i] % 4 == 0 && aligned(gy[i], 4 * esz)) layers[i].vec |= kVecIn;
        if (ch[i] % 4 == 0 && aligned(g[i], 4 * esz)) layers[i].vec |= kVecOut;
        tiles += hw[i] == 1 ? tp * tc : batch[i] * tc * tp;
    }
    const size_t need = kfac_grad_rows_workspace_size(n);
    if (workspace == nullptr || !aligned(workspace, kAlign) || workspace_bytes < need) return KFAC_ERR_WORKSPACE;
    Carver c(workspace);
    GradRowsLayer* dev = static_cast<GradRowsLayer*>(c.take(sizeof(GradRowsLayer) * n));
    hipError_t e = upload_table(dev, layers.data(), sizeof(GradRowsLayer) * n, stream);
    if (e != hipSuccess) return KFAC_ERR_HIP;
    return hip_status(launch_grad_rows(dev, n, tiles, dtype == KFAC_BF16, scale, stream));
}

size_t kfac_grad_matrix_workspace_size(int n) {
    if (n < 1 || n > KFAC_MAX_COUNT) return 0;
    Carver c(nullptr);
    c.take(sizeof(GradMatLayer) * n);
    return c.used;
}

kfac_status_t kfac_grad_matrix(int n, float* const* wgrad, float* const* bgrad, const int64_t* d_out,
                               const int64_t* d_in, float* const* mat, kfac_pack_dir_t dir,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (n < 1 || n > KFAC_MAX_COUNT || wgrad == nullptr || d_out == nullptr || d_in == nullptr || mat == nullptr)
        return KFAC_ERR_INVALID_VALUE;
    if (dir != KFAC_PACK && dir != KFAC_UNPACK) return KFAC_ERR_INVALID_VALUE;
    std::vector<GradMatLayer> layers(n);
    int64_t chunks = 0;
    for (int i = 0; i < n; ++i) {
        float* b = bgrad ? bgrad[i] : nullptr;
        if (wgrad[i] == nullptr || mat[i] == nullptr || !aligned(wgrad[i], 4) || !aligned(mat[i], 4) ||
            (b != nullptr && !aligned(b, 4)))
            return KFAC_ERR_INVALID_VALUE;
        if (d_out[i] < 1 || d_in[i] < 1) return KFAC_ERR_INVALID_VALUE;
        const int64_t cols = d_in[i] + (b ? 1 : 0);
        layers[i] = GradMatLayer{wgrad[i], b, mat[i], d_out[i], d_in[i], chunks, cols};
        chunks += ceil_div(d_out[i] * cols, kGradMatChunk);
    }
    const size_t need = kfac_grad_matrix_workspace_size(n);
    if (workspace == nullptr || !aligned(workspace, kAlign) || workspace_bytes < need) return KFAC_ERR_WORKSPACE;
    Carver c(workspace);
    GradMatLayer* dev = static_cast<GradMatLayer*>(c.take(sizeof(GradMatLayer) * n));
    hipError_t e = upload_table(dev, layers.data(), sizeof(GradMatLayer) * n, stream);
    if (e != hipSuccess) return KFAC_ERR_HIP;
    return hip_status(launch_grad_matrix(dev, n, chunks, dir == KFAC_PACK, stream));
}

}  // extern "C"
