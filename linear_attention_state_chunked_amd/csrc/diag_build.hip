// Diagonal (GLA) and scalar (RetNet, Mamba2) segment build.
//
// With A_t = diag(alpha_t) the segment's transition and zero-start state have closed
// forms (decaying families of the HYPIC news article's linear-layer paragraph):
//   T = diag(exp(G_n)),   S(C|0) = sum_t diag(exp(G_n - G_t)) k_t v_t^T,
// with G_t = sum_{j<=t} log alpha_j per channel (one value for the scalar kind).
// S is one dense contraction over the segment's tokens: K~^T V with
// K~[t][c] = k_t[c] exp(G_n[c] - G_t[c]).  Chunks are visited from the end of the
// segment backwards so the decay exponent is a running suffix sum; K~ and V are
// staged in LDS (f16, contraction axis in accumulator order) and contracted on the
// matrix cores, the d x d state staying in accumulators.
#include "device_common.hpp"
#include "kernels.hpp"

namespace hypic {

template <int D, class Op>
__global__ __launch_bounds__(512) void diag_build_kernel(DiagArgs a) {
    using E = typename Op::elem;
    constexpr int PAD = 16 / (int)sizeof(E);
    constexpr int RS = 64 + PAD;
    constexpr int NT = 512;
    constexpr int KS = Op::KS, KH = Op::KH;
    constexpr int TILES = (D / 32) * (D / 32);
    constexpr int TPW = (TILES + 7) / 8;  // tiles per wave
    constexpr int NP = NT / D;            // token parts per chunk
    constexpr int TP = kChunk / NP;       // tokens per part
    __shared__ __align__(16) E sKd[D * RS];   // K~^T: [c][t]
    __shared__ __align__(16) E sVt[D * RS];   // V^T : [d][t]
    __shared__ float sR[D];                   // running suffix sum per channel
    __shared__ float sPart[NT];               // per-part decay sums
    __shared__ float sMax;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, l32 = lane & 31;
    const bool in_bf16 = a.in_bf16 != 0;
    const long long N = a.n_tokens;

    const int task = a.order ? a.order[blockIdx.x] : blockIdx.x;
    const int per_seg = a.n_batch * a.h_v;
    const int seg = task / per_seg;
    const int rem = task - seg * per_seg;
    const int b = rem / a.h_v, h = rem - (rem / a.h_v) * a.h_v;
    const int hk = (h * a.h_k) / a.h_v;
    const long long start = a.seg_start[seg];
    const int len = a.seg_len[seg];
    const long long chain = (long long)seg * a.n_batch * a.h_v + (long long)b * a.h_v + h;

    floatx16 acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) acc[i] = zero16();
    if (tid < D) sR[tid] = 0.f;
    __syncthreads();

    const int nchunk = (len + kChunk - 1) / kChunk;
    for (int ci = nchunk - 1; ci >= 0; --ci) {
        const int c0 = ci * kChunk;
        const int valid = min(kChunk, len - c0);
        const long long tok0 = start + c0;
        // decayed keys: thread (c, p) handles channel c over token part p of the chunk;
        // part offsets (suffix sums of later parts) are exchanged through LDS.
        {
            const int c = tid % D, p = tid / D;
            float kv[TP], la[TP];
            float tot = 0.f;
#pragma unroll
            for (int u = 0; u < TP; ++u) {
                const int t = p * TP + u;
                kv[u] = 0.f;
                la[u] = 0.f;
                if (t < valid) {
                    const long long row = (b * N + tok0 + t);
                    const long long ki = (row * a.h_k + hk) * D + c;
                    kv[u] = in_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.k)[ki])
                                    : reinterpret_cast<const float*>(a.k)[ki];
                    la[u] = a.scalar ? a.log_alpha[row * a.h_v + h] : a.log_alpha[(row * a.h_v + h) * D + c];
                }
                tot += la[u];
            }
            sPart[p * D + c] = tot;
            __syncthreads();
            float run = sR[c];
            for (int q = p + 1; q < NP; ++q) run += sPart[q * D + c];
#pragma unroll
            for (int u = TP - 1; u >= 0; --u) {
                sKd[c * RS + acc_pos(p * TP + u)] = Op::cvt(kv[u] * expf(run));
                run += la[u];
            }
            __syncthreads();
            if (p == 0) {
                float r = sR[c];
                for (int q = 0; q < NP; ++q) r += sPart[q * D + c];
                sR[c] = r;
            }
        }
        // values, transposed
        for (int i = tid; i < kChunk * (D / 8); i += NT) {
            const int t = i / (D / 8), d0 = 8 * (i % (D / 8));
            float x[8];
            if (t < valid) load8(a.v, ((b * N + tok0 + t) * a.h_v + h) * D + d0, in_bf16, x);
            else {
#pragma unroll
                for (int u = 0; u < 8; ++u) x[u] = 0.f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) sVt[(d0 + u) * RS + acc_pos(t)] = Op::cvt(x[u]);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int tile = wave * TPW + i;
            if (tile >= TILES) break;
            const int tr = tile / (D / 32), tc = tile % (D / 32);
#pragma unroll
            for (int kk = 0; kk < kChunk / KS; ++kk) {
                const auto fa = Op::load(sKd + (32 * tr + l32) * RS + KS * kk + KH * half);
                const auto fb = Op::load(sVt + (32 * tc + l32) * RS + KS * kk + KH * half);
                acc[i] = Op::mma(fa, fb, acc[i]);
            }
        }
        __syncthreads();
    }

    float* dS = a.S + chain * D * D;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int tile = wave * TPW + i;
        if (tile >= TILES) break;
        const int tr = tile / (D / 32), tc = tile % (D / 32);
#pragma unroll
        for (int j = 0; j < 16; ++j) dS[(32 * tr + acc_row(half, j)) * D + 32 * tc + l32] = acc[i][j];
    }
    if (a.T_hat) {
        // T = exp(G_n) per channel, written as T_hat * 2^e with max T_hat in (0.5, 1]
        if (wave == 0) {
            float m = -INFINITY;
            for (int c = lane; c < (a.scalar ? 1 : D); c += 64) m = fmaxf(m, sR[c]);
            m = wave_max(m);
            if (lane == 0) sMax = m;
        }
        __syncthreads();
        const float l2e = 1.4426950408889634f;
        const int e = (int)ceilf(sMax * l2e);
        if (a.scalar) {
            if (tid == 0) a.T_hat[chain] = exp2f(sR[0] * l2e - (float)e);
        } else if (tid < D) {
            a.T_hat[chain * D + tid] = exp2f(sR[tid] * l2e - (float)e);
        }
        if (tid == 0) a.T_exp[chain] = e;
    }
}

hipError_t launch_diag_build(const DiagArgs& a, int d, hipStream_t s) {
    const int grid = a.n_tasks;
    if (d == 128) {
        if (a.in_bf16) hipLaunchKernelGGL((diag_build_kernel<128, OpF16>), dim3(grid), dim3(512), 0, s, a);
        else hipLaunchKernelGGL((diag_build_kernel<128, OpF32>), dim3(grid), dim3(512), 0, s, a);
    } else if (d == 64) {
        if (a.in_bf16) hipLaunchKernelGGL((diag_build_kernel<64, OpF16>), dim3(grid), dim3(512), 0, s, a);
        else hipLaunchKernelGGL((diag_build_kernel<64, OpF32>), dim3(grid), dim3(512), 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace hypic
