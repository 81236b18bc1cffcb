// Matrix-core rate reference.  Every workgroup (four waves) runs rounds of
// four independent products on register operands and no memory traffic
// besides one float per wave at the end, so the figure it gives is what the
// matrix cores sustain on this part under its own clock and power limits.
// The HBM-bound stages have the copy kernel as their measured reference;
// this is the counterpart for the matrix-core-bound ones.  It is no stage of
// the path: its entry point lives here, apart from the others.
//
// Operands are fixed pseudo-random values in [-1, 1) with random signs (the
// data a product sees changes its power draw, and so the clock), so the
// accumulators take a random walk and stay finite.
#include "device_common.h"
#include "kfac.h"

namespace kfac {
namespace {

constexpr int kRateBf16 = 0, kRateF64 = 1, kRateF32 = 2;

typedef __bf16 bf16x8r __attribute__((ext_vector_type(8)));

// An integer hash with good avalanche (the published "lowbias32" finaliser
// of C. Wellons' hash-prospector), for the operands only.
__device__ __forceinline__ uint32_t mix(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// A float in [-1, 1) from 24 random bits and a random sign.
__device__ __forceinline__ float operand(uint32_t h) {
    const float m = (float)(h >> 8) * (1.0f / 16777216.0f);
    return (h & 1u) ? -m : m;
}

// Two workgroups per CU (two waves per SIMD).  The occupancy hint also
// keeps the accumulators in VGPRs: without it the compiler put the float64
// products' accumulators in AGPRs and copied them to VGPRs and back on
// every round of the loop.
template <int KIND>
__global__ __launch_bounds__(256, 2) void matrix_rate_kernel(int64_t iters, float* __restrict__ sink) {
    const uint32_t g = blockIdx.x * 256u + threadIdx.x;
    float total = 0.0f;
    if constexpr (KIND == kRateBf16) {
        bf16x8r a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = (__bf16)operand(mix(g * 16u + i));
            b[i] = (__bf16)operand(mix(g * 16u + 8 + i));
        }
        floatx16 acc[4] = {};
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) total += acc[j][r];
    } else if constexpr (KIND == kRateF64) {
        const double a = operand(mix(2u * g)), b = operand(mix(2u * g + 1u));
        doublex4 acc[4] = {};
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) total += (float)acc[j][r];
    } else {
        const float a = operand(mix(2u * g)), b = operand(mix(2u * g + 1u));
        floatx16 acc[4] = {};
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) total += acc[j][r];
    }
    // one float per wave keeps every wave's products
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = total;
}

// Flops of one round of one wave: four products.
double matrix_rate_flops_per_round(int kind) {
    // four products per wave and round
    switch (kind) {
        case kRateBf16: return 4.0 * 32 * 32 * 16 * 2;
        case kRateF64: return 4.0 * 16 * 16 * 4 * 2;
        default: return 4.0 * 32 * 32 * 2 * 2;
    }
}

hipError_t launch_matrix_rate(int kind, int64_t iters, int blocks, float* sink, hipStream_t stream) {
    switch (kind) {
        case kRateBf16:
            hipLaunchKernelGGL(matrix_rate_kernel<kRateBf16>, dim3(blocks), dim3(256), 0, stream, iters, sink);
            break;
        case kRateF64:
            hipLaunchKernelGGL(matrix_rate_kernel<kRateF64>, dim3(blocks), dim3(256), 0, stream, iters, sink);
            break;
        default:
            hipLaunchKernelGGL(matrix_rate_kernel<kRateF32>, dim3(blocks), dim3(256), 0, stream, iters, sink);
            break;
    }
    return hipGetLastError();
}

}  // namespace
}  // namespace kfac

extern "C" kfac_status_t kfac_matrix_rate(kfac_rate_kind_t kind, int64_t iters, int blocks, float* sink,
                                          double* flops, hipStream_t stream) {
    using namespace kfac;
    if (kind != KFAC_RATE_BF16 && kind != KFAC_RATE_F64 && kind != KFAC_RATE_F32) return KFAC_ERR_INVALID_VALUE;
    if (iters < 1 || iters > (int64_t(1) << 24) || blocks < 1 || blocks > 65536) return KFAC_ERR_INVALID_VALUE;
    if (sink == nullptr || reinterpret_cast<uintptr_t>(sink) % 4 != 0) return KFAC_ERR_INVALID_VALUE;
    const int k = kind == KFAC_RATE_BF16 ? kRateBf16 : (kind == KFAC_RATE_F64 ? kRateF64 : kRateF32);
    if (flops != nullptr) *flops = matrix_rate_flops_per_round(k) * (double)iters * 4.0 * (double)blocks;
    return launch_matrix_rate(k, iters, blocks, sink, stream) == hipSuccess ? KFAC_OK : KFAC_ERR_HIP;
}
