// RoPE state re-rotation of cached elements moved to a new absolute offset.
//
// A segment cached with keys rotated at positions p + t and reused at p + delta + t has
// keys R k, R = R(delta) block-diagonal with 2 x 2 rotations by delta * theta_i on the
// rotated channel pairs, theta_i = base^(-2i / rotary_dim).  Its per-token transitions
// become R A_t R^T and its writes R k v^T, so the cached state becomes R S and the
// transition R T R^T (the alignment patch for RoPE variants of the HYPIC news article's
// linear-layer paragraph; the transition_rope mode of the HYPIC project README).
//
// Every output entry depends only on the 2 x 2 (T) or 2 x 1 (S) block of the input at the
// same channel pairs, so each thread reads a block and writes it back: the update may run
// in place.  One workgroup per (element, chain); consecutive threads take consecutive
// column pairs (T) or columns (S), so the loads of a wave are row segments.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace hypic {

// channel pair p: (a, b) and whether it rotates; pairs p >= rotary_dim/2 are the
// remaining channels two by two, left alone
struct PairMap {
    int h, rd, interleaved;
    __device__ __forceinline__ int a(int p) const {
        if (interleaved) return 2 * p;
        return p < h ? p : rd + 2 * (p - h);
    }
    __device__ __forceinline__ int b(int p) const {
        if (interleaved) return 2 * p + 1;
        return p < h ? p + h : rd + 2 * (p - h) + 1;
    }
};

template <int D>
__global__ __launch_bounds__(256) void rerotate_kernel(RotArgs r) {
    constexpr int NP = D / 2;
    __shared__ float sc[NP], ss[NP];
    const int chain = blockIdx.x, e = blockIdx.y, tid = threadIdx.x;
    const long long delta = r.delta[e];
    const PairMap pm{r.rotary_dim / 2, r.rotary_dim, r.interleaved};
    if (tid < NP) {
        float c = 1.f, s = 0.f;
        if (tid < pm.h) {
            // the angle in double: delta reaches 1e5 and more, where a float angle is off by ~1e-2
            const double theta = exp2(-2.0 * tid / r.rotary_dim * r.log2_base);
            double sd, cd;
            sincos((double)delta * theta, &sd, &cd);
            c = (float)cd;
            s = (float)sd;
        }
        sc[tid] = c;
        ss[tid] = s;
    }
    __syncthreads();
    const long long blk = (long long)(r.elem0 + e) * r.n_chain + chain;
    const long long DD = (long long)D * D;
    // S' = R S: rows a, b of each pair
    {
        const float* Si = r.S_in + blk * DD;
        float* So = r.S_out + blk * DD;
        for (int i = tid; i < NP * D; i += 256) {
            const int p = i / D, col = i - p * D;
            const int ra = pm.a(p), rb = pm.b(p);
            const float x = Si[ra * D + col], y = Si[rb * D + col];
            const float c = sc[p], s = ss[p];
            So[ra * D + col] = c * x - s * y;
            So[rb * D + col] = s * x + c * y;
        }
    }
    if (!r.dense) return;
    // T' = R T R^T: block (P, Q) -> R_P [T_aA T_aB; T_bA T_bB] R_Q^T
    const float* Ti = r.T_in + blk * DD;
    float* To = r.T_out + blk * DD;
    for (int i = tid; i < NP * NP; i += 256) {
        const int P = i / NP, Q = i - P * NP;
        const int ra = pm.a(P), rb = pm.b(P), ca = pm.a(Q), cb = pm.b(Q);
        const float t00 = Ti[ra * D + ca], t01 = Ti[ra * D + cb], t10 = Ti[rb * D + ca], t11 = Ti[rb * D + cb];
        const float cP = sc[P], sP = ss[P], cQ = sc[Q], sQ = ss[Q];
        // rows: R_P X
        const float u00 = cP * t00 - sP * t10, u01 = cP * t01 - sP * t11;
        const float u10 = sP * t00 + cP * t10, u11 = sP * t01 + cP * t11;
        // columns: X R_Q^T, whose column pair mixes as (x_A, x_B) -> (c x_A - s x_B, s x_A + c x_B)
        To[ra * D + ca] = cQ * u00 - sQ * u01;
        To[ra * D + cb] = sQ * u00 + cQ * u01;
        To[rb * D + ca] = cQ * u10 - sQ * u11;
        To[rb * D + cb] = sQ * u10 + cQ * u11;
    }
}

hipError_t launch_rerotate(const RotArgs& r, int d, int n_elem, hipStream_t s) {
    const dim3 grid(r.n_chain, n_elem);
    if (d == 128) hipLaunchKernelGGL(rerotate_kernel<128>, grid, dim3(256), 0, s, r);
    else if (d == 64) hipLaunchKernelGGL(rerotate_kernel<64>, grid, dim3(256), 0, s, r);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace hypic
