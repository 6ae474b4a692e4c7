// Matrix-core rate probe (libhypic_probe): back-to-back v_mfma_f32_32x32x16_f16 products on register
// operands, 2 waves per SIMD with 4 independent accumulators each, so that the matrix cores never wait
// for an operand or a result.  Wave 0 of each workgroup reads the core-clock counter and the 100 MHz
// real-time counter around its products.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hypic_probe.h"

namespace {

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8;     // 2 per SIMD
constexpr int kAcc = 4;       // independent products in flight per wave
constexpr double kFlopsPerProduct = 32.0 * 32.0 * 16.0 * 2.0;

__global__ __launch_bounds__(kWaves * 64) void mfma_probe_kernel(float* sink, int64_t* clocks, int iters) {
    const int tid = threadIdx.x, lane = tid & 63;
    halfx8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(0.001f * (float)(lane + i));
        b[i] = (_Float16)(0.001f * (float)(lane - i));
    }
    floatx16 acc[kAcc];
#pragma unroll
    for (int k = 0; k < kAcc; ++k)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[k][j] = 0.f;
    __syncthreads();
    const int64_t c0 = (int64_t)__builtin_amdgcn_s_memtime();
    const int64_t r0 = (int64_t)__builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < kAcc; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[k], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kAcc; ++k)
#pragma unroll
        for (int j = 0; j < 16; ++j) s += acc[k][j];
    const int64_t c1 = (int64_t)__builtin_amdgcn_s_memtime();
    const int64_t r1 = (int64_t)__builtin_amdgcn_s_memrealtime();
    sink[(size_t)blockIdx.x * (kWaves * 64) + tid] = s;
    if (tid == 0) {
        clocks[2 * (size_t)blockIdx.x] = c1 - c0;
        clocks[2 * (size_t)blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace

extern "C" double hypic_probe_mfma_f16_flops(int n_groups, int iters) {
    return (double)n_groups * kWaves * (double)iters * kAcc * kFlopsPerProduct;
}

extern "C" int hypic_probe_mfma_f16(int n_groups, int iters, float* sink, int64_t* clocks,
                                    hypic_probe_stream_t stream) {
    if (n_groups < 1 || iters < 1 || !sink || !clocks) return -1;
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(n_groups), dim3(kWaves * 64), 0,
                       reinterpret_cast<hipStream_t>(stream), sink, clocks, iters);
    return (int)hipGetLastError();
}
