// Seam advance for short seams (w <= 16 tokens): the seam window of the HYPIC news
// article's seam-window paragraph, in the closed low-rank form of one chunk.
//
// For the w seam tokens (local index a = 0..w-1) of one (seam, batch, value head):
//   G_a = sum_{t<=a} log alpha_t,  gamma_a = e^{G_a},  Gamma = gamma_{w-1}
//   L   = strictly-lower(beta_a e^{G_a - G_b} k_a.k_b),  Tg = (I + L)^-1 diag(beta)
//   M   = diag(Gamma/gamma) Tg diag(gamma),   N = diag(Gamma/gamma) Tg
//   T_seam = Gamma I - K^T M K,               S_seam = K^T N V          (from (I, 0))
//   S_out  = Gamma S_in + K^T (N V - M K S_in)                         (= T_seam S_in + S_seam)
//   o      = diag(gamma) Q S_in + Mq (Tg V - Tg diag(gamma) K S_in),
//            Mq = lower(e^{G_a - G_b} q_a.k_b) including the diagonal   (o_t = S_t^T q_t)
// Every d x d output is a rank-w update, so the work is a handful of w x w matrices and
// one pass over the d x d blocks: thread (column j, part p) owns rows
// [p*RPT, (p+1)*RPT) of column j of S_in / S_out / T / S_seam, so every global access
// of a d x d block is a coalesced row segment and no d x d block touches LDS; the
// w x d factors live in LDS.
// Arithmetic is fp32 throughout (VALU).
#include "device_common.hpp"
#include "kernels.hpp"

namespace hypic {

// W <= 8: at most 128 VGPRs (four waves per SIMD) and about 37 KB of LDS, so several
// workgroups share a compute unit and hide each other's latency-bound w x w steps.
template <int D, int W, bool IN_BF16>
__global__ __launch_bounds__(4 * D, W <= 8 ? 4 : 1) void seam_kernel(SeamArgs a) {
    constexpr int NT = 4 * D;
    constexpr int TPC = 4;               // threads per column
    constexpr int RPT = D / TPC;         // rows per thread
    constexpr int G8 = D / 8;            // 8-element groups per row
    static_assert(W * G8 <= NT, "one 8-element group per thread per tensor");
    __shared__ __align__(16) float sK[W][D + 4];   // rows 16-byte aligned: 4-float LDS reads
    __shared__ __align__(16) float sV[W][D];
    __shared__ __align__(16) float sQ[W][D + 4];
    __shared__ float sL[W][W + 1];       // L, later M
    __shared__ float sMq[W][W + 1];
    __shared__ float sTg[W][W + 1];
    __shared__ float sG[W], sGam[W], sScl[W], sBeta[W];
    __shared__ float sU[W][D];           // Tg V
    __shared__ float sRT[W][D];          // M K, later P = K S_in
    __shared__ float sP[W][D];           // partials, later Q S_in
    __shared__ float sQS[W][D];          // partials
    __shared__ float sY[W][D];           // partials, later U - Tg diag(gamma) P
    __shared__ float sZ[W][D];           // partials, later RS - M P
    __shared__ float sRed[NT / 64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per_seam = a.n_batch * a.h_v;
    const int task = blockIdx.x;
    const int s = task / per_seam;
    const int rem = task - s * per_seam;
    const int b = rem / a.h_v;
    const int h = rem - b * a.h_v;
    const int hk = (h * a.h_k) / a.h_v;
    const long long tok0 = seg_start(a.seg, s);
    const int w = seg_len(a.seg, s);
    const long long chain = (long long)b * a.h_v + h;
    const long long DD = (long long)D * D;
    const bool want_o = a.o != nullptr;
    const bool want_in = a.S_in != nullptr && (want_o || a.S_out != nullptr);
    // thread (column j, part) owns rows [i0, i0 + RPT) of column j of every d x d block
    const int j = tid % D, part = tid / D, i0 = part * RPT;
    float sin_run[RPT];

    // ---- seam tokens: k, v (and q) rows, optionally L2-normalised; gates
    {
        const int t = tid / G8, d0 = 8 * (tid % G8);
        if (tid < W * G8) {
            float xk[8], xv[8], xq[8];
            if (t < w) {
                const long long tok = (long long)b * a.n_tokens + tok0 + t;
                load8(a.k, (tok * a.h_k + hk) * D + d0, IN_BF16, xk);
                load8(a.v, (tok * a.h_v + h) * D + d0, IN_BF16, xv);
                if (want_o) load8(a.q, (tok * a.h_k + hk) * D + d0, IN_BF16, xq);
                else
#pragma unroll
                    for (int u = 0; u < 8; ++u) xq[u] = 0.f;
            } else {
#pragma unroll
                for (int u = 0; u < 8; ++u) xk[u] = xv[u] = xq[u] = 0.f;
            }
            if (a.qk_l2norm) {
                float sk = 0.f, sq = 0.f;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    sk += xk[u] * xk[u];
                    sq += xq[u] * xq[u];
                }
                // a token row's G8 pieces sit on G8 adjacent lanes: DPP sums, no LDS round trip
                sk = group_sum<G8>(sk);
                sq = group_sum<G8>(sq);
                const float ck = sk > 0.f ? 1.f / sqrtf(sk) : 0.f;
                const float cq = sq > 0.f ? 1.f / sqrtf(sq) : 0.f;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    xk[u] *= ck;
                    xq[u] *= cq;
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                sK[t][d0 + u] = xk[u];
                sV[t][d0 + u] = xv[u];
                sQ[t][d0 + u] = xq[u];
            }
        }
        if (wave == 0) {
            const bool ok = lane < w;
            const long long gi = ((long long)b * a.n_tokens + tok0 + lane) * a.h_v + h;
            const float la = ok ? a.log_alpha[gi] : 0.f;
            const float bt = ok ? a.beta[gi] : 0.f;
            const float G = wave_scan_dpp(la);
            const float Gl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G), w > 0 ? w - 1 : 0));
            if (lane < W) {
                sG[lane] = G;
                sGam[lane] = expf(G);
                sScl[lane] = expf(Gl - G);
                sBeta[lane] = bt;
            }
        }
    }
    __syncthreads();
    const float Gamma = w > 0 ? sGam[w - 1] : 1.f;
    // this thread's run of S_in, loaded before the w x w steps so that its HBM latency hides
    // behind them (after the token loads, whose registers are free by now)
    if (want_in) {
        const float* Sin = a.S_in + s * a.in_stride + chain * DD + j;
#pragma unroll
        for (int ii = 0; ii < RPT; ++ii) sin_run[ii] = Sin[(long long)(i0 + ii) * D];
    }

    // ---- w x w: L (strictly lower) and Mq (lower with diagonal).  Every thread takes part:
    //      each dot product of length D is split over SUBS adjacent lanes (D / SUBS elements
    //      each, 4-float LDS reads) and summed with DPP lane permutations.
    {
        constexpr int SUBS = NT / 64;        // 8 (D = 128), 4 (D = 64)
        constexpr int EPS = D / SUBS;        // 16
        static_assert((W * W) % 64 == 0 && (SUBS == 4 || SUBS == 8), "pair tiling");
        const int sub = tid % SUBS;
        for (int p0 = 0; p0 < W * W; p0 += 64) {
            const int p = p0 + tid / SUBS;
            const int r = p / W, c = p % W;
            const bool on = r < w && c <= r;
            float dk = 0.f, dq = 0.f;
            if (on) {
#pragma unroll
                for (int e = 0; e < EPS; e += 4) {
                    const float4 kr = *reinterpret_cast<const float4*>(&sK[r][sub * EPS + e]);
                    const float4 kc = *reinterpret_cast<const float4*>(&sK[c][sub * EPS + e]);
                    const float4 qr = *reinterpret_cast<const float4*>(&sQ[r][sub * EPS + e]);
                    dk += kr.x * kc.x + kr.y * kc.y + kr.z * kc.z + kr.w * kc.w;
                    dq += qr.x * kc.x + qr.y * kc.y + qr.z * kc.z + qr.w * kc.w;
                }
            }
            dk += dpp_perm<0xb1>(dk);            // quad_perm [1,0,3,2]
            dq += dpp_perm<0xb1>(dq);
            dk += dpp_perm<0x4e>(dk);            // quad_perm [2,3,0,1]
            dq += dpp_perm<0x4e>(dq);
            if constexpr (SUBS == 8) {
                dk += dpp_perm<0x141>(dk);       // row_half_mirror: the other quad of the 8
                dq += dpp_perm<0x141>(dq);
            }
            if (sub == 0) {
                const float g = on ? expf(sG[r] - sG[c]) : 0.f;
                sL[r][c] = (c < r) ? sBeta[r] * g * dk : 0.f;
                sMq[r][c] = g * dq;
            }
        }
    }
    __syncthreads();
    // ---- Tg = (I + L)^-1 diag(beta): column c by forward substitution (one lane each)
    if (tid < W) {
        const int c = tid;
        float y[W];
#pragma unroll
        for (int r = 0; r < W; ++r) {
            float acc = (r == c) ? sBeta[r] : 0.f;
#pragma unroll
            for (int q = 0; q < r; ++q) acc -= sL[r][q] * y[q];
            y[r] = (r < c) ? 0.f : acc;
        }
#pragma unroll
        for (int r = 0; r < W; ++r) sTg[r][c] = y[r];
    }
    __syncthreads();
    // M = diag(Gamma/gamma) Tg diag(gamma) into sL (L is no longer needed)
    for (int p = tid; p < W * W; p += NT) {
        const int r = p / W, c = p % W;
        sL[r][c] = sScl[r] * sTg[r][c] * sGam[c];
    }
    __syncthreads();

    // ---- w x d factors, thread (column j, part) computes rows [RW*part, RW*part + RW):
    //      U = Tg V, RT = M K  (RS = diag(Gamma/gamma) U is formed where it is used)
    constexpr int RW = W / TPC;
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
        const int r = RW * part + rr;
        float u = 0.f, rt = 0.f;
#pragma unroll
        for (int c = 0; c < W; ++c) {
            u += sTg[r][c] * sV[c][j];
            rt += sL[r][c] * sK[c][j];
        }
        sU[r][j] = u;
        sRT[r][j] = rt;
    }
    __syncthreads();

    if (a.T_hat || a.S_seam) {
        const long long ob = ((long long)s * per_seam + chain) * DD;
        if (a.T_hat) {
            // T_seam[:, j] = Gamma e_j - K^T RT[:, j]
            float tv[RPT];
#pragma unroll
            for (int ii = 0; ii < RPT; ++ii) tv[ii] = (i0 + ii == j) ? Gamma : 0.f;
#pragma unroll 4
            for (int r = 0; r < W; ++r) {
                const float rt = sRT[r][j];
#pragma unroll
                for (int ii = 0; ii < RPT; ++ii) tv[ii] -= sK[r][i0 + ii] * rt;
            }
            float m = 0.f;
#pragma unroll
            for (int ii = 0; ii < RPT; ++ii) m = fmaxf(m, fabsf(tv[ii]));
            m = wave_max(m);
            if (lane == 0) sRed[wave] = m;
            __syncthreads();
            float mm = sRed[0];
#pragma unroll
            for (int q = 1; q < NT / 64; ++q) mm = fmaxf(mm, sRed[q]);
            const int e = exp2_of(mm);
            const float sc = ldexpf(1.f, -e);
            float* dst = a.T_hat + ob + j;
#pragma unroll
            for (int ii = 0; ii < RPT; ++ii) dst[(long long)(i0 + ii) * D] = tv[ii] * sc;
            if (tid == 0) a.T_exp[(long long)s * per_seam + chain] = e;
        }
        if (a.S_seam) {
            // S_seam[:, j] = K^T RS[:, j]
            float sv[RPT];
#pragma unroll
            for (int ii = 0; ii < RPT; ++ii) sv[ii] = 0.f;
#pragma unroll 4
            for (int r = 0; r < W; ++r) {
                const float z = sScl[r] * sU[r][j];
#pragma unroll
                for (int ii = 0; ii < RPT; ++ii) sv[ii] += sK[r][i0 + ii] * z;
            }
            float* dst = a.S_seam + ob + j;
#pragma unroll
            for (int ii = 0; ii < RPT; ++ii) dst[(long long)(i0 + ii) * D] = sv[ii];
        }
    }

    if (want_in) {
        float (&sv)[RPT] = sin_run;
        // P = K S_in[:, j] and QS = Q S_in[:, j]: partial sums over this thread's rows in
        // four LDS slots (one per part), summed in a fixed order (bitwise reproducible)
        auto slot = [&](int q) -> float (*)[D] { return q == 0 ? sP : q == 1 ? sQS : q == 2 ? sY : sZ; };
        static_assert(TPC == 4, "four partial slots");
        float PQ[2][W];
#pragma unroll 4
        for (int r = 0; r < W; ++r) {
            float p = 0.f, q = 0.f;
#pragma unroll
            for (int ii = 0; ii < RPT; ++ii) {
                p += sK[r][i0 + ii] * sv[ii];
                q += sQ[r][i0 + ii] * sv[ii];
            }
            PQ[0][r] = p;
            PQ[1][r] = q;
        }
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            if (pass == 1 && !want_o) break;
#pragma unroll
            for (int r = 0; r < W; ++r) slot(part)[r][j] = PQ[pass][r];
            __syncthreads();
            // this thread's rows of the total: P into sRT (free now), QS into sP
#pragma unroll
            for (int rr = 0; rr < RW; ++rr) {
                const int r = RW * part + rr;
                float acc = 0.f;
#pragma unroll
                for (int q = 0; q < TPC; ++q) acc += slot(q)[r][j];
                if (pass == 0) sRT[r][j] = acc;
                else sP[r][j] = acc;
            }
            __syncthreads();
        }
        // Y = U - Tg diag(gamma) P (for o) and Z = RS - M P (for S_out), rows of this thread
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            const int r = RW * part + rr;
            float y = sU[r][j], z = sScl[r] * sU[r][j];
#pragma unroll
            for (int c = 0; c < W; ++c) {
                const float pc = sRT[c][j];
                y -= sTg[r][c] * sGam[c] * pc;
                z -= sL[r][c] * pc;
            }
            sY[r][j] = y;
            sZ[r][j] = z;
        }
        __syncthreads();
        if (want_o) {
            // o[t][j] = gamma_t QS[t] + sum_{c <= t} Mq[t][c] Y[c]
#pragma unroll
            for (int rr = 0; rr < RW; ++rr) {
                const int t = RW * part + rr;
                if (t < w) {
                    float acc = sGam[t] * sP[t][j];
#pragma unroll
                    for (int c = 0; c < W; ++c) acc += sMq[t][c] * sY[c][j];
                    const long long oi = (((long long)b * a.n_tokens + tok0 + t) * a.h_v + h) * D + j;
                    if (a.out_bf16) reinterpret_cast<uint16_t*>(a.o)[oi] = f32_to_bf16(acc);
                    else reinterpret_cast<float*>(a.o)[oi] = acc;
                }
            }
        }
        if (a.S_out) {
            // S_out[:, j] = Gamma S_in[:, j] + K^T Z[:, j]  (alias-safe: own elements only)
#pragma unroll
            for (int ii = 0; ii < RPT; ++ii) sv[ii] *= Gamma;
#pragma unroll 4
            for (int r = 0; r < W; ++r) {
                const float z = sZ[r][j];
#pragma unroll
                for (int ii = 0; ii < RPT; ++ii) sv[ii] += sK[r][i0 + ii] * z;
            }
            float* dst = a.S_out + s * a.out_stride + chain * DD + j;
#pragma unroll
            for (int ii = 0; ii < RPT; ++ii) dst[(long long)(i0 + ii) * D] = sv[ii];
        }
    } else {
        if (a.S_out) {
            // S_in = 0: S_out = S_seam = K^T RS
            float sv[RPT];
#pragma unroll
            for (int ii = 0; ii < RPT; ++ii) sv[ii] = 0.f;
#pragma unroll 4
            for (int r = 0; r < W; ++r) {
                const float z = sScl[r] * sU[r][j];
#pragma unroll
                for (int ii = 0; ii < RPT; ++ii) sv[ii] += sK[r][i0 + ii] * z;
            }
            float* dst = a.S_out + s * a.out_stride + chain * DD + j;
#pragma unroll
            for (int ii = 0; ii < RPT; ++ii) dst[(long long)(i0 + ii) * D] = sv[ii];
        }
        if (want_o) {
            // S_in = 0: o = Mq U
#pragma unroll
            for (int rr = 0; rr < RW; ++rr) {
                const int t = RW * part + rr;
                if (t < w) {
                    float acc = 0.f;
#pragma unroll
                    for (int c = 0; c < W; ++c) acc += sMq[t][c] * sU[c][j];
                    const long long oi = (((long long)b * a.n_tokens + tok0 + t) * a.h_v + h) * D + j;
                    if (a.out_bf16) reinterpret_cast<uint16_t*>(a.o)[oi] = f32_to_bf16(acc);
                    else reinterpret_cast<float*>(a.o)[oi] = acc;
                }
            }
        }
    }
}

template <int D, int W>
static hipError_t launch_seam_w(const SeamArgs& a, hipStream_t s) {
    const dim3 grid(a.n_tasks);
    if (a.in_bf16) hipLaunchKernelGGL((seam_kernel<D, W, true>), grid, dim3(4 * D), 0, s, a);
    else hipLaunchKernelGGL((seam_kernel<D, W, false>), grid, dim3(4 * D), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_seam(const SeamArgs& a, int d, int w_max, hipStream_t s) {
    if (w_max > kSeamShort) return hipErrorInvalidValue;
    if (d == 128) return w_max <= 8 ? launch_seam_w<128, 8>(a, s) : launch_seam_w<128, kSeamShort>(a, s);
    if (d == 64) return w_max <= 8 ? launch_seam_w<64, 8>(a, s) : launch_seam_w<64, kSeamShort>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace hypic
