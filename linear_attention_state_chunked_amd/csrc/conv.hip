// Depthwise causal convolution with the state carried across a segment boundary
// (conv-state warm-up, HYPIC news article's linear-layer paragraph).
//
// y_t[c] = act(bias[c] + sum_j w[c][j] * xx[t + j][c]), xx = (W-1 carried rows) ++ x.
// Every output is independent: one thread computes 8 consecutive channels of a block
// of 8 consecutive tokens, HBM-bound streaming with 16-byte loads; the first thread
// block of a segment also emits state_out.
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

// grid: x = (token blocks of kConvT tokens of the longest segment) x (channel groups of
// 8), y = segment, z = batch.  A thread keeps its 8 channels' taps in registers and
// slides a window of W rows over its token block, so each input row is loaded once.
constexpr int kConvT = 8;

__global__ __launch_bounds__(256) void conv_kernel(ConvArgs a) {
    const int groups = a.channels / 8;
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int seg = blockIdx.y, b = blockIdx.z;
    const int tb = (int)(i / groups);
    const int c0 = 8 * (int)(i - (long long)tb * groups);
    const int len = seg_len(a.seg, seg);
    const int nblk = max((len + kConvT - 1) / kConvT, 1);   // block 0 also writes state_out
    if (tb >= nblk) return;
    const long long start = seg_start(a.seg, seg);
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

    const int t0 = tb * kConvT;
    if (t0 < len) {
        const float* wb = a.weight + ((long long)b * C + c0) * kConvW;  // this batch entry's taps
        float w[8][kConvW];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float4 wv = *reinterpret_cast<const float4*>(wb + u * kConvW);
            w[u][0] = wv.x;
            w[u][1] = wv.y;
            w[u][2] = wv.z;
            w[u][3] = wv.w;
        }
        float bias[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) bias[u] = a.bias ? a.bias[(long long)b * C + c0 + u] : 0.f;
        float win[kConvW][8];
#pragma unroll
        for (int j = 0; j < kConvW - 1; ++j) fetch(t0 + j, win[j]);
#pragma unroll
        for (int k = 0; k < kConvT; ++k) {
            const int t = t0 + k;
            if (t < len) {
                fetch(t + kConvW - 1, win[(k + kConvW - 1) % kConvW]);
                float y[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    float acc = bias[u];
#pragma unroll
                    for (int j = 0; j < kConvW; ++j) acc += w[u][j] * win[(k + j) % kConvW][u];
                    y[u] = a.silu ? acc / (1.f + expf(-acc)) : acc;
                }
                store8(a.y, ((long long)b * a.n_tokens + start + t) * C + c0, a.out_bf16 != 0, y);
            }
        }
    }
    if (a.state_out && tb == 0) {
        // state_out row t = xx[len + t]
#pragma unroll
        for (int t = 0; t < kConvW - 1; ++t) {
            float x[8];
            fetch(len + t, x);
            store8(a.state_out, (((long long)seg * a.n_batch + b) * (kConvW - 1) + t) * C + c0, in_bf16, x);
        }
    }
}

hipError_t launch_conv(const ConvArgs& a, long long max_span, hipStream_t s) {
    const long long blocks = (max_span + kConvT - 1) / kConvT;
    const long long threads = (blocks > 0 ? blocks : 1) * (a.channels / 8);
    const dim3 grid((unsigned)((threads + 255) / 256), a.n_seg, a.n_batch);
    hipLaunchKernelGGL(conv_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace hypic
