// Composition of cached segments: S <- T_i S + S_i in request order.
//
// The composition law S(C1.C2) = T(C2) S(C1) + S(C2) of the HYPIC news article's
// linear-layer paragraph, applied element by element.  One kernel serves every
// compose mode: a launch is a grid of (chain, block); block `blk` folds a contiguous
// run of elements starting from (I, init_S[blk]) and writes its end state, optionally
// its aggregate transition and the state entering each element.  FOLD is one block
// per chain; SCAN is a blocked reduce (aggregates), a fold over the block aggregates,
// and a re-fold that writes the per-element states.
//
// Dense kind: each wave owns 32 columns of X = [T | S] in matrix-core accumulators
// and computes T_i X with f16 hi/lo operand splits (three products, ~22-bit operand
// precision) after scaling its column block by an exact power of two; T_i is staged in
// LDS as hi/lo f16 with its contraction axis in accumulator order.
// Diagonal / scalar kinds: elementwise, one thread per state entry stripe.
#include "device_common.hpp"
#include "kernels.hpp"

namespace hypic {

__device__ __forceinline__ void split_hilo(const floatx16& x, int st, halfx8& hi, halfx8& lo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float v = x[8 * st + i];
        const _Float16 h = (_Float16)v;
        hi[i] = h;
        lo[i] = (_Float16)(v - (float)h);
    }
}

template <int D, bool WITH_T>
__global__ __launch_bounds__((WITH_T ? 2 : 1) * D * 2) void fold_dense_kernel(FoldArgs a) {
    constexpr int NWS = D / 32;                     // S waves
    constexpr int NW = (WITH_T ? 2 : 1) * NWS;
    constexpr int NB = D / 32;
    constexpr int RS = D + 8;
    __shared__ __align__(16) _Float16 sThi[D * RS];
    __shared__ __align__(16) _Float16 sTlo[D * RS];
    __shared__ int sE;
    __shared__ int sEw[8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, l32 = lane & 31;
    const bool t_wave = WITH_T && wave < NWS;
    const int col0 = (t_wave ? wave : (WITH_T ? wave - NWS : wave)) * 32;
    const int chain = blockIdx.x, blk = blockIdx.y;
    const int e0 = blk * a.per_block;
    const int e1 = min(a.n_elem, e0 + a.per_block);
    const long long DD = (long long)D * D;

    floatx16 X[NB];
    if (t_wave) {
#pragma unroll
        for (int xb = 0; xb < NB; ++xb)
#pragma unroll
            for (int j = 0; j < 16; ++j) X[xb][j] = (32 * xb + acc_row(half, j) == col0 + l32) ? 1.f : 0.f;
    } else if (a.init_S) {
        const float* src = a.init_S + ((long long)blk * a.n_chain + chain) * DD;
#pragma unroll
        for (int xb = 0; xb < NB; ++xb)
#pragma unroll
            for (int j = 0; j < 16; ++j) X[xb][j] = src[(32 * xb + acc_row(half, j)) * D + col0 + l32];
    } else {
#pragma unroll
        for (int xb = 0; xb < NB; ++xb) X[xb] = zero16();
    }
    int ew = 0;

    for (int el = e0; el < e1; ++el) {
        const int slot = a.slot ? a.slot[el] : el;
        const long long so = (long long)slot * a.n_chain + chain;
        if (a.prefix && !t_wave) {
            float* dst = a.prefix + ((long long)el * a.n_chain + chain) * DD;
#pragma unroll
            for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                for (int j = 0; j < 16; ++j) dst[(32 * xb + acc_row(half, j)) * D + col0 + l32] = X[xb][j];
        }
        const float* Si = a.S + so * DD;
        if (a.naive) {
            if (!t_wave) {
#pragma unroll
                for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) X[xb][j] += Si[(32 * xb + acc_row(half, j)) * D + col0 + l32];
            }
            continue;
        }
        // stage T_i as hi/lo f16, rows = output rows, columns in accumulator order
        const float* Ti = a.T_hat + so * DD;
        for (int i = tid; i < D * D / 4; i += NW * 64) {
            const int r = (4 * i) / D, c = (4 * i) % D;
            const float4 v = reinterpret_cast<const float4*>(Ti)[i];
            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const _Float16 hv = (_Float16)vv[u];
                sThi[r * RS + acc_pos(c + u)] = hv;
                sTlo[r * RS + acc_pos(c + u)] = (_Float16)(vv[u] - (float)hv);
            }
        }
        if (tid == 0) sE = a.T_exp[so];
        __syncthreads();
        const int ei = sE;
        // scale this wave's column block to max |x| in [0.5, 1) before splitting
        float m = 0.f;
#pragma unroll
        for (int xb = 0; xb < NB; ++xb)
#pragma unroll
            for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(X[xb][j]));
        const int sx = exp2_of(wave_max(m));
        halfx8 bh[NB][2], bl[NB][2];
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
            floatx16 xs;
#pragma unroll
            for (int j = 0; j < 16; ++j) xs[j] = ldexpf(X[kb][j], -sx);
            split_hilo(xs, 0, bh[kb][0], bl[kb][0]);
            split_hilo(xs, 1, bh[kb][1], bl[kb][1]);
        }
#pragma unroll
        for (int ob = 0; ob < NB; ++ob) {
            floatx16 acc = zero16();
#pragma unroll
            for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    const int off = (32 * ob + l32) * RS + 32 * kb + 16 * half + 8 * st;
                    const halfx8 ah = *reinterpret_cast<const halfx8*>(sThi + off);
                    const halfx8 al = *reinterpret_cast<const halfx8*>(sTlo + off);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bh[kb][st], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bl[kb][st], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh[kb][st], acc, 0, 0, 0);
                }
            if (t_wave) {
                X[ob] = acc;  // T columns: exponent tracked separately
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    X[ob][j] = ldexpf(acc[j], sx + ei) + Si[(32 * ob + acc_row(half, j)) * D + col0 + l32];
            }
        }
        if (t_wave) {
            // X holds T_i * (X * 2^-sx): exponent += sx + ei, then renormalise
            float mm = 0.f;
#pragma unroll
            for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                for (int j = 0; j < 16; ++j) mm = fmaxf(mm, fabsf(X[xb][j]));
            const int e = exp2_of(wave_max(mm));
#pragma unroll
            for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                for (int j = 0; j < 16; ++j) X[xb][j] = ldexpf(X[xb][j], -e);
            ew += sx + ei + e;
        }
        __syncthreads();
    }

    if (WITH_T && a.out_T) {
        if (t_wave && lane == 0) sEw[wave] = ew;
        __syncthreads();
        if (t_wave) {
            int emax = sEw[0];
            for (int w = 1; w < NWS; ++w) emax = max(emax, sEw[w]);
            float* dst = a.out_T + ((long long)blk * a.n_chain + chain) * DD;
#pragma unroll
            for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    dst[(32 * xb + acc_row(half, j)) * D + col0 + l32] = ldexpf(X[xb][j], ew - emax);
            if (tid == 0) a.out_e[(long long)blk * a.n_chain + chain] = emax;
        }
    }
    if (!t_wave && a.out_S) {
        float* dst = a.out_S + ((long long)blk * a.n_chain + chain) * DD;
#pragma unroll
        for (int xb = 0; xb < NB; ++xb)
#pragma unroll
            for (int j = 0; j < 16; ++j) dst[(32 * xb + acc_row(half, j)) * D + col0 + l32] = X[xb][j];
    }
}

// Diagonal (T a d_k vector) and scalar (T one value) kinds: elementwise.
template <int D>
__global__ __launch_bounds__(256) void fold_diag_kernel(FoldArgs a) {
    constexpr int NT = 256;
    constexpr int PER = D * D / NT;
    __shared__ float sT[D];
    __shared__ float sRed[4];
    __shared__ int sEi;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int chain = blockIdx.x, blk = blockIdx.y;
    const bool scalar = a.kind == 2;
    const int e0 = blk * a.per_block;
    const int e1 = min(a.n_elem, e0 + a.per_block);
    const long long DD = (long long)D * D;
    const int tlen = scalar ? 1 : D;

    float x[PER];
    if (a.init_S) {
        const float* src = a.init_S + ((long long)blk * a.n_chain + chain) * DD;
#pragma unroll
        for (int r = 0; r < PER; ++r) x[r] = src[tid + NT * r];
    } else {
#pragma unroll
        for (int r = 0; r < PER; ++r) x[r] = 0.f;
    }
    float tv = 1.f;  // thread tid < tlen owns T[tid]
    int te = 0;
    for (int el = e0; el < e1; ++el) {
        const int slot = a.slot ? a.slot[el] : el;
        const long long so = (long long)slot * a.n_chain + chain;
        if (a.prefix) {
            float* dst = a.prefix + ((long long)el * a.n_chain + chain) * DD;
#pragma unroll
            for (int r = 0; r < PER; ++r) dst[tid + NT * r] = x[r];
        }
        const float* Si = a.S + so * DD;
        if (a.naive) {
#pragma unroll
            for (int r = 0; r < PER; ++r) x[r] += Si[tid + NT * r];
            continue;
        }
        if (tid < tlen) sT[tid] = a.T_hat[so * tlen + tid];
        if (tid == 0) sEi = a.T_exp[so];
        __syncthreads();
        const int ei = sEi;
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const int row = (tid + NT * r) / D;
            x[r] = ldexpf((scalar ? sT[0] : sT[row]) * x[r], ei) + Si[tid + NT * r];
        }
        if (a.out_T) {
            // running product of transitions, renormalised by the block max
            if (tid < tlen) tv *= sT[tid];
            float m = tid < tlen ? fabsf(tv) : 0.f;
            m = wave_max(m);
            if (lane == 0) sRed[wave] = m;
            __syncthreads();
            const float mm = fmaxf(fmaxf(sRed[0], sRed[1]), fmaxf(sRed[2], sRed[3]));
            const int e = exp2_of(mm);
            tv = ldexpf(tv, -e);
            te += ei + e;
        }
        __syncthreads();
    }
    if (a.out_S) {
        float* dst = a.out_S + ((long long)blk * a.n_chain + chain) * DD;
#pragma unroll
        for (int r = 0; r < PER; ++r) dst[tid + NT * r] = x[r];
    }
    if (a.out_T) {
        if (tid < tlen) a.out_T[((long long)blk * a.n_chain + chain) * tlen + tid] = tv;
        if (tid == 0) a.out_e[(long long)blk * a.n_chain + chain] = te;
    }
}

hipError_t launch_fold(const FoldArgs& a, int d, int with_T, hipStream_t s) {
    const dim3 grid(a.n_chain, a.n_block);
    if (a.kind == 0 && !a.naive) {
        if (d == 128) {
            if (with_T) hipLaunchKernelGGL((fold_dense_kernel<128, true>), grid, dim3(512), 0, s, a);
            else hipLaunchKernelGGL((fold_dense_kernel<128, false>), grid, dim3(256), 0, s, a);
        } else if (d == 64) {
            if (with_T) hipLaunchKernelGGL((fold_dense_kernel<64, true>), grid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((fold_dense_kernel<64, false>), grid, dim3(128), 0, s, a);
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        // naive addition of any kind, and the diagonal / scalar kinds
        if (d == 128) hipLaunchKernelGGL((fold_diag_kernel<128>), grid, dim3(256), 0, s, a);
        else if (d == 64) hipLaunchKernelGGL((fold_diag_kernel<64>), grid, dim3(256), 0, s, a);
        else return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace hypic
