// Depthwise causal convolution with the state carried across a segment boundary
// (conv-state warm-up, HYPIC news article's linear-layer paragraph).
//
// y_t[c] = act(bias[c] + sum_j w[c][j] * xx[t + j][c]), xx = (W-1 carried rows) ++ x.
// Every output is independent, so one thread computes 8 consecutive channels of one
// token: HBM-bound streaming with 16-byte loads, the W-1 earlier rows re-read
// through the cache.  Threads of a segment's first W-1 tokens also emit state_out.
#include "device_common.hpp"
#include "kernels.hpp"

namespace hypic {

constexpr int kConvW = 4;

__device__ __forceinline__ void store8(void* base, long long idx, bool bf16, const float (&y)[8]) {
    if (bf16) {
        uint4 w;
        w.x = (uint32_t)f32_to_bf16(y[0]) | ((uint32_t)f32_to_bf16(y[1]) << 16);
        w.y = (uint32_t)f32_to_bf16(y[2]) | ((uint32_t)f32_to_bf16(y[3]) << 16);
        w.z = (uint32_t)f32_to_bf16(y[4]) | ((uint32_t)f32_to_bf16(y[5]) << 16);
        w.w = (uint32_t)f32_to_bf16(y[6]) | ((uint32_t)f32_to_bf16(y[7]) << 16);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(base) + idx) = w;
    } else {
        float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + idx);
        p[0] = make_float4(y[0], y[1], y[2], y[3]);
        p[1] = make_float4(y[4], y[5], y[6], y[7]);
    }
}

// grid: x = token blocks of the longest segment (x channel groups), y = segment, z = batch
__global__ __launch_bounds__(256) void conv_kernel(ConvArgs a) {
    const int groups = a.channels / 8;
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int seg = blockIdx.y, b = blockIdx.z;
    const int t = (int)(i / groups);
    const int c0 = 8 * (int)(i - (long long)t * groups);
    const int len = a.seg_len[seg];
    const int span = max(len, kConvW - 1);
    if (t >= span) return;
    const long long start = a.seg_start[seg];
    const bool in_bf16 = a.in_bf16 != 0;
    const long long C = a.channels;
    int srow = -1;
    if (a.state_in) srow = a.state_index ? a.state_index[seg] : seg;

    // input row r of xx (r = 0..W-2 carried state, r >= W-1 the segment's tokens)
    auto fetch = [&](int r, float (&x)[8]) {
        if (r >= kConvW - 1) {
            load8(a.x, ((long long)b * a.n_tokens + start + (r - (kConvW - 1))) * C + c0, in_bf16, x);
        } else if (srow >= 0) {
            load8(a.state_in, (((long long)srow * a.n_batch + b) * (kConvW - 1) + r) * C + c0, in_bf16, x);
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = 0.f;
        }
    };

    if (t < len) {
        const float* wb = a.weight + (long long)b * C * kConvW;  // this batch entry's taps
        float y[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) y[u] = a.bias ? a.bias[(long long)b * C + c0 + u] : 0.f;
#pragma unroll
        for (int j = 0; j < kConvW; ++j) {
            float x[8];
            fetch(t + j, x);
#pragma unroll
            for (int u = 0; u < 8; ++u) y[u] += wb[(c0 + u) * kConvW + j] * x[u];
        }
        if (a.silu) {
#pragma unroll
            for (int u = 0; u < 8; ++u) y[u] = y[u] / (1.f + expf(-y[u]));
        }
        store8(a.y, ((long long)b * a.n_tokens + start + t) * C + c0, a.out_bf16 != 0, y);
    }
    if (a.state_out && t < kConvW - 1) {
        // state_out row t = xx[len + t]
        float x[8];
        fetch(len + t, x);
        store8(a.state_out, (((long long)seg * a.n_batch + b) * (kConvW - 1) + t) * C + c0, in_bf16, x);
    }
}

hipError_t launch_conv(const ConvArgs& a, long long max_span, hipStream_t s) {
    const long long threads = max_span * (a.channels / 8);
    const dim3 grid((unsigned)((threads + 255) / 256), a.n_seg, a.n_batch);
    hipLaunchKernelGGL(conv_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace hypic
