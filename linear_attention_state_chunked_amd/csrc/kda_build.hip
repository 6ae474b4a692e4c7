// Segment build of the per-channel gated delta rule (KDA family):
//   A_t = diag(alpha_t) (I - beta_t k_t k_t^T),   S_t = A_t S_{t-1} + beta_t k_t v_t^T,
// T_C the ordered product of the A_t (a dense d x d transition, so cached KDA segments
// compose with the dense composition law of the HYPIC news article's linear-layer
// paragraph, which names KDA among the families), S(C|0) the zero-start state.
//
// Token-sequential, float32 vector arithmetic.  Four threads own column j of X = [T | S]
// (a quarter of its d rows each, in registers; lanes l, l ^ 16, l ^ 32, l ^ 48 of one wave);
// columns evolve independently under X <- A_t X + [0 | w_t], so a token needs only the sum of
// the four partial dot products u_j = k_t^T X_j (two lane exchanges), then
//   X_rj <- alpha_r X_rj - alpha_r k_r beta u_j (+ k_r beta v_j for the state columns).
// Four threads per column give 16 waves per workgroup with d/4 rows each (107 VGPRs), so
// every SIMD issues from four waves (one thread per column ran at 290 registers, one wave
// per SIMD: 2.3 ms against 1.3 ms for the 16 x 512-token, 32-head layer).
// The per-channel gates make the chunked WY/UT form need per-channel exponentials of gate
// differences inside a chunk (overflow-prone in f16 operands); the token form has none.
// Tokens are staged 16 at a time in LDS (k, alpha, alpha k, beta, v) and read as
// broadcasts.  Each T column carries its own power-of-two exponent (column scaling
// commutes with left multiplication); the exponents are aligned once at the end.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace hypic {

template <int D, bool WITH_T, bool IN_BF16>
__global__ __launch_bounds__((WITH_T ? 8 : 4) * D) void kda_build_kernel(KdaArgs a) {
    constexpr int NT = (WITH_T ? 8 : 4) * D;
    constexpr int DH = D / 4;   // rows per thread
    constexpr int CH = 16;
    __shared__ __align__(16) float sK[CH][D];
    __shared__ __align__(16) float sA[CH][D];
    __shared__ __align__(16) float sAK[CH][D];
    __shared__ __align__(16) float sV[CH][D];
    __shared__ float sB[CH];
    __shared__ int sE[NT / 64];

    const int tid = threadIdx.x;
    const int per_seg = a.n_batch * a.h_v;
    const int task = task_at(a.seg, blockIdx.x, per_seg);
    const int seg = task / per_seg;
    const int rem = task - seg * per_seg;
    const int b = rem / a.h_v, h = rem - (rem / a.h_v) * a.h_v;
    const int hk = (h * a.h_k) / a.h_v;
    const long long start = seg_start(a.seg, seg);
    const int len = seg_len(a.seg, seg);
    const long long N = a.n_tokens;
    // wave w holds columns 32 w .. 32 w + 31 of [T | S]; lane l holds rows hf DH .. of column
    // 32 w + (l & 31), hf = l >> 5
    const int lane = tid & 63, wv = tid >> 6, hf = lane >> 4;
    const int gcol = 16 * wv + (lane & 15);
    const bool t_col = WITH_T && gcol < D;
    const int col = (WITH_T && gcol >= D) ? gcol - D : gcol;
    const int r0 = hf * DH;

    float X[DH];
#pragma unroll
    for (int r = 0; r < DH; ++r) X[r] = (t_col && r0 + r == col) ? 1.f : 0.f;
    int ex = 0;

    for (int c0 = 0; c0 < len; c0 += CH) {
        const int nt = min(CH, len - c0);
        __syncthreads();  // the previous chunk's tokens are consumed
        for (int i = tid; i < CH * D; i += NT) {
            const int t = i / D, r = i - t * D;
            float kv = 0.f, al = 1.f, vv = 0.f;
            if (t < nt) {
                const long long row = (long long)b * N + start + c0 + t;
                const long long ki = (row * a.h_k + hk) * D + r;
                const long long vi = (row * a.h_v + h) * D + r;
                if (IN_BF16) {
                    kv = bf16_to_f32(reinterpret_cast<const uint16_t*>(a.k)[ki]);
                    vv = bf16_to_f32(reinterpret_cast<const uint16_t*>(a.v)[vi]);
                } else {
                    kv = reinterpret_cast<const float*>(a.k)[ki];
                    vv = reinterpret_cast<const float*>(a.v)[vi];
                }
                al = expf(a.log_alpha[vi]);
            }
            sK[t][r] = kv;
            sA[t][r] = al;
            sAK[t][r] = al * kv;
            sV[t][r] = vv;
        }
        if (tid < CH) {
            const long long row = (long long)b * N + start + c0 + tid;
            sB[tid] = tid < nt ? a.beta[row * a.h_v + h] : 0.f;
        }
        __syncthreads();
        for (int t = 0; t < nt; ++t) {
            // k^T X_j as 8 independent partial sums (one dependent chain of d FMAs would
            // stall a wave that has its SIMD to itself)
            float up[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) up[i] = 0.f;
#pragma unroll
            for (int r = 0; r < DH; ++r) up[r & 7] = fmaf(sK[t][r0 + r], X[r], up[r & 7]);
            float u = ((up[0] + up[1]) + (up[2] + up[3])) + ((up[4] + up[5]) + (up[6] + up[7]));
            u += __shfl_xor(u, 16, 64);   // the other row quarters of this column
            u += __shfl_xor(u, 32, 64);
            const float bt = sB[t];
            const float w = bt * u;
            if (t_col) {
#pragma unroll
                for (int r = 0; r < DH; ++r) X[r] = fmaf(-sAK[t][r0 + r], w, sA[t][r0 + r] * X[r]);
            } else {
                const float wvv = bt * sV[t][col];
#pragma unroll
                for (int r = 0; r < DH; ++r)
                    X[r] = fmaf(sK[t][r0 + r], wvv, fmaf(-sAK[t][r0 + r], w, sA[t][r0 + r] * X[r]));
            }
        }
        if (t_col) {
            // this column's largest magnitude back into [0.5, 1)
            float m = 0.f;
#pragma unroll
            for (int r = 0; r < DH; ++r) m = fmaxf(m, fabsf(X[r]));
            m = fmaxf(m, __shfl_xor(m, 16, 64));   // all row quarters
            m = fmaxf(m, __shfl_xor(m, 32, 64));
            const int e = exp2_of(m);
            if (e != 0) {
#pragma unroll
                for (int r = 0; r < DH; ++r) X[r] = ldexpf(X[r], -e);
                ex += e;
            }
        }
    }

    const long long chain = (long long)b * a.h_v + h;
    if (WITH_T) {
        // align the T columns to one exponent: the largest over the columns
        int em = t_col ? ex : INT32_MIN;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) em = max(em, __shfl_xor(em, o, 64));
        if ((tid & 63) == 0) sE[tid >> 6] = em;
        __syncthreads();
        int emax = sE[0];
        for (int w = 1; w < D / 16; ++w) emax = max(emax, sE[w]);   // the waves of T columns
        if (t_col) {
            float* dst = a.T_hat + ((long long)seg * a.n_batch * a.h_v + chain) * D * D + (long long)r0 * D + col;
#pragma unroll
            for (int r = 0; r < DH; ++r) dst[(long long)r * D] = ldexpf(X[r], ex - emax);
            if (tid == 0) a.T_exp[(long long)seg * a.n_batch * a.h_v + chain] = emax;
        }
    }
    if (!t_col) {
        float* dst = a.S + ((long long)seg * a.n_batch * a.h_v + chain) * D * D + (long long)r0 * D + col;
#pragma unroll
        for (int r = 0; r < DH; ++r) dst[(long long)r * D] = X[r];
    }
}

template <int D, bool WITH_T>
static hipError_t launch_kda_d(const KdaArgs& a, hipStream_t s) {
    constexpr int nt = (WITH_T ? 8 : 4) * D;
    if (a.in_bf16) hipLaunchKernelGGL((kda_build_kernel<D, WITH_T, true>), dim3(a.n_tasks), dim3(nt), 0, s, a);
    else hipLaunchKernelGGL((kda_build_kernel<D, WITH_T, false>), dim3(a.n_tasks), dim3(nt), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_kda_build(const KdaArgs& a, int d, hipStream_t s) {
    const bool t = a.T_hat != nullptr;
    if (d == 128) return t ? launch_kda_d<128, true>(a, s) : launch_kda_d<128, false>(a, s);
    if (d == 64) return t ? launch_kda_d<64, true>(a, s) : launch_kda_d<64, false>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace hypic
