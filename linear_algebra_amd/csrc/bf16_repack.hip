// bfloat16 factor inputs of odd width: copied to a pitch that is a multiple
// of 64 elements before the factor GEMM.  A row of odd width starts on a
// 2-byte boundary every other row, and the 16-byte copies that stage GEMM
// slabs straight into LDS only read from 4-byte boundaries; after the copy
// every row starts on a 128-byte cache line and the factor takes the copy
// path, each 256-byte row segment of a slab then covering two whole lines
// (from a 16-byte boundary it touches three).
#include "device_common.h"
#include "internal.h"

namespace kfac {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Repacks a bf16 input whose rows do not all start on 4-byte boundaries
// (odd width) into a copy whose pitch is a multiple of 64 elements (rows on
// 128-byte lines), columns past the width zero.  Each thread writes one
// 16-byte group of 8 elements of one row, read as 20 bytes from the 4-byte
// boundary at or below it and shifted into place.  Each layer has its own
// range of workgroups, so a workgroup's rows all belong to one layer and
// one buffer descriptor (rebased at its first row) covers them.
__global__ __launch_bounds__(256) void repack_bf16_kernel(const RepackLayer* __restrict__ layers, int n,
                                                          int64_t blocks) {
    const int64_t blk = blockIdx.x;
    if (blk >= blocks) return;
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (layers[mid].block_begin <= blk) lo = mid; else hi = mid - 1;
    }
    const RepackLayer& R = layers[lo];
    const int64_t upr = R.pitch / 8;                              // groups per row
    const int64_t u0 = (blk - R.block_begin) * 256;
    const int64_t u = u0 + threadIdx.x;
    if (u >= R.rows * upr) return;
    const int64_t r0 = u0 / upr, r = u / upr;
    const int q = (int)(u % upr);
    // rows [r0, r0 + nr) are all this workgroup can touch
    const int64_t nr = min(R.rows - r0, (int64_t)(256 / upr + 2));
    const uintptr_t p = reinterpret_cast<uintptr_t>(R.src) + (uintptr_t)(r0 * R.d) * 2;
    const uintptr_t p4 = p & ~(uintptr_t)3;
    const uint32_t delta = (uint32_t)(p - p4);
    const int bytes = (int)((delta + 2 * nr * R.d + 3) & ~(int64_t)3);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(p4), (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
    const uint32_t off = delta + 2u * (uint32_t)((r - r0) * R.d + 8 * q);
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rs, off & ~3u, 0, 0);
    const uint32_t w4 = __builtin_amdgcn_raw_buffer_load_b32(rs, (off & ~3u) + 16, 0, 0);
    const uint32_t sh = off & 2u;
    u32x4 v;
    v[0] = __builtin_amdgcn_alignbyte(w[1], w[0], sh);
    v[1] = __builtin_amdgcn_alignbyte(w[2], w[1], sh);
    v[2] = __builtin_amdgcn_alignbyte(w[3], w[2], sh);
    v[3] = __builtin_amdgcn_alignbyte(w4, w[3], sh);
    // columns past the width (the next row's first elements) become zero
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int c = 8 * q + 2 * k;
        if (c >= R.d) v[k] = 0u;
        else if (c + 1 >= R.d) v[k] &= 0xFFFFu;
    }
    *reinterpret_cast<u32x4*>(R.dst + r * R.pitch + 8 * q) = v;
}

}  // namespace

hipError_t launch_repack_bf16(const RepackLayer* layers, int n, int64_t blocks, hipStream_t stream) {
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(repack_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, layers, n, blocks);
    return hipGetLastError();
}

}  // namespace kfac
