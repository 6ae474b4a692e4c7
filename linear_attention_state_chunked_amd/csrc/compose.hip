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
// Dense kind: each wave owns 32 columns of S (and, for the composed transition, of
// T) in matrix-core accumulators and computes T_i X with f16 hi/lo operand splits
// (three products, ~22-bit operand precision) after scaling its column block by an
// exact power of two (the column maximum uses the NaN-propagating three-input maximum
// with |.| modifiers); T_i is staged row-major in LDS as hi/lo f16 by loader waves in
// two column halves, each as soon as the compute waves are done with that half of the
// previous element (LDS counters, no workgroup barrier per element).  A fold that carries the
// running state alone can instead split each chain's columns over d/16 workgroups
// (fold_split_kernel), for few chains on many compute units.
// Diagonal / scalar kinds: elementwise, one thread per state entry stripe.
#include <mutex>

#include "device_common.hpp"
#include "kernels.hpp"

namespace hypic {

// Scratch of the allocation-free compose entry point: one fixed array per device, held from
// module load until the process ends.  Host code never passes `scratch` itself (on the host
// the name only stands in for the symbol); it asks the runtime for the device address once
// per device and hands that to the kernels.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* cached[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!cached[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        cached[dev] = p;
    }
    *ptr = cached[dev];
    return hipSuccess;
}

// Sticky status word of the compose kernels (see take_compose_status): a bounded wait that ran
// out sets it.
__device__ unsigned int g_compose_status;

hipError_t take_compose_status(unsigned* out) {
    unsigned v = 0;
    const unsigned z = 0;
    hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_compose_status), sizeof v, 0, hipMemcpyDeviceToHost);
    if (e == hipSuccess && v) e = hipMemcpyToSymbol(HIP_SYMBOL(g_compose_status), &z, sizeof z, 0, hipMemcpyHostToDevice);
    *out = v;
    return e;
}

// One arrival per wave on an LDS counter, after the wave's earlier LDS accesses.
__device__ __forceinline__ void fold_arrive(int* cnt, int lane) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Bounded wait until an LDS counter reaches target; a wait that runs out sets the status word
// and goes on, so the kernel still ends.
__device__ __forceinline__ void fold_wait(int* cnt, int target) {
    int spins = 0;
    while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
        if (++spins > (1 << 20)) {
            __hip_atomic_fetch_or(&g_compose_status, kStatusWaitExpired, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ void split_hilo(const floatx16& x, int st, float scale, halfx8& hi, halfx8& lo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float v = x[8 * st + i] * scale;
        const _Float16 h = (_Float16)v;
        hi[i] = h;
        lo[i] = (_Float16)(v - (float)h);
    }
}

// A fragment of T_i for output row `row`, contraction block kb, step st: the 8
// contraction indices a lane half h supplies in accumulator order are
// 32kb + 16st + 4h + {0..3} and 32kb + 16st + 8 + 4h + {0..3}, two 8-byte runs of
// the row-major staged tile.
__device__ __forceinline__ halfx8 t_frag(const _Float16* base) {
    typedef _Float16 half4 __attribute__((ext_vector_type(4)));
    const half4 x = *reinterpret_cast<const half4*>(base);
    const half4 y = *reinterpret_cast<const half4*>(base + 8);
    halfx8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = x[i];
        r[4 + i] = y[i];
    }
    return r;
}

// Dense kind.  One workgroup per (chain, element block, role); role 0 composes S,
// role 1 (launched only when the composed transition is wanted) composes T.  D/32
// compute waves each keep 32 columns of the running S (or T) in accumulators; D/16
// loader waves hold the next element's (T_i, and for role 0 S_i) in registers, loaded
// from HBM while the current element is multiplied, and write them into LDS (T_i as
// hi/lo f16, S_i as fp32, row-major) between two workgroup barriers.
// SEAM: the fused warm path.  Loader wave t also loads seam token t of the next element
// (q, k, v rows, gates).  The seam window (w <= 8 tokens) is applied in the one-chunk form of
// the gated delta rule: while the compute waves multiply element el, the loader waves turn
// the window of el + 1 into its factors (the w x w gram and output mask, Tg = (I + L)^-1
// diag(beta) by forward substitution, -Tg diag(gamma) K, diag(gamma) Q and K^T as hi/lo f16
// tiles).  Before each element's product the compute waves then advance their accumulator-
// resident columns on the matrix cores: Z = Tg V - Tg diag(gamma) K S, O = diag(gamma) Q S +
// Mq Z (the window's outputs o_t = S_t^T q_t), S <- Gamma S + K^T diag(Gamma / gamma) Z.
template <int D, bool SEAM>
__global__ __launch_bounds__(D * 6) void fold_dense_kernel(FoldArgs a) {
    constexpr int NB = D / 32;                        // compute waves
    constexpr int NLT = 2 * NB * 64;                  // loader threads
    constexpr int RS = D + 8;                         // staged row stride (halves)
    constexpr int TPL = D * D / (4 * NLT);            // float4 of T_i per loader thread
    static_assert(TPL * 4 * NLT == D * D, "staging split");
    constexpr int RSS = D + 4;                        // staged S_i row stride (floats)
    __shared__ __align__(16) _Float16 sT[2][D * RS];      // hi, lo
    __shared__ __align__(16) float sS[D * RSS];
    __shared__ int sE;
    __shared__ int sEw[NB];
    constexpr int WS = SEAM ? kFusedSeamMax : 1;
    // seam window of the staged element (w <= kFusedSeamMax tokens), in the one-chunk form of the gated
    // delta rule (rows = window tokens; row WS of each w-row tile stays zero for the padded rows of the
    // 32-row matrix-core operands):
    //   G_t = sum_{s<=t} log alpha_s, gamma_t = e^{G_t}, Gamma = gamma_{w-1}
    //   L = strictly-lower(beta_t e^{G_t - G_s} k_t.k_s),  Tg = (I + L)^-1 diag(beta)
    //   Z = Tg V - Tg diag(gamma) K S,  S' = Gamma S + K^T diag(Gamma / gamma) Z
    //   O = diag(gamma) Q S + Mq Z,     Mq = lower(e^{G_t - G_s} q_t.k_s), diagonal included
    constexpr int RW = D + 4;                       // row stride (halves) of the w x D operand tiles
    constexpr int WK = SEAM ? D : 1;
    __shared__ __align__(16) _Float16 sWh[WS + 1][RW], sWl[WS + 1][RW];   // -Tg diag(gamma) K, hi / lo
    __shared__ __align__(16) _Float16 sQh[WS + 1][RW], sQl[WS + 1][RW];   // diag(gamma) Q, hi / lo
    __shared__ __align__(16) _Float16 sKTh[WK][8], sKTl[WK][8];           // K^T, hi / lo
    __shared__ __align__(16) _Float16 sTh[WS + 1][8], sTl[WS + 1][8];     // Tg, hi / lo
    __shared__ __align__(16) _Float16 sMh[WS + 1][8], sMl[WS + 1][8];     // Mq, hi / lo
    __shared__ __align__(16) float sKf[WS][D + 4];  // the window's keys (fp32, for the w x w products)
    __shared__ __align__(16) float sVs[WS][D];      // the window's values
    __shared__ float sLf[WS][WS], sTgf[WS][WS];     // L and Tg (fp32)
    __shared__ float sGb[WS][2];                    // log alpha, beta
    __shared__ float sGv[WS], sR[WS], sGam;         // gamma_t, Gamma / gamma_t, Gamma
    __shared__ int sW;                              // seam tokens of the staged element
    // hand-off counters: T_i column half A, half B and S_i staged (one arrival per loader wave),
    // then consumed (one per compute wave)
    __shared__ int sC[9];

    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool loader = wave >= NB;
    const bool t_role = blockIdx.z == 1;
    const int chain = blockIdx.x, blk = blockIdx.y;
    const int e0 = blk * a.per_block;
    const int e1 = min(a.n_elem, e0 + a.per_block);
    const long long DD = (long long)D * D;
    auto elem = [&](int el) __attribute__((always_inline)) -> long long {
        const int sl = a.slot ? a.slot[el] : el;
        return (long long)sl * a.n_chain + chain;
    };

    constexpr int NLW = NLT / 64;                     // loader waves
    if (tid < 9) sC[tid] = 0;
    if constexpr (SEAM) {
        // the zero rows of the window's operand tiles
        for (int i = tid; i < RW; i += D * 6) {
            sWh[WS][i] = sWl[WS][i] = sQh[WS][i] = sQl[WS][i] = (_Float16)0.f;
            if (i < 8) sTh[WS][i] = sTl[WS][i] = sMh[WS][i] = sMl[WS][i] = (_Float16)0.f;
        }
    }
    __syncthreads();
    if (loader) {
        const int lt = tid - NB * 64;
        typedef float f4 __attribute__((ext_vector_type(4)));
        // T_i by column halves: float4 r of half h of loader thread lt is row (lt + NLT r) / (D / 8),
        // columns h D / 2 + 4 ((lt + NLT r) % (D / 8)) .. + 3
        constexpr int TPH = TPL / 2;
        f4 th[2][TPH], ts[TPL];
        int ei = 0;
        // seam tokens lw, lw + NLW, ... (loader wave lw): lane l holds channels l, l + 64, ...
        constexpr int NLW = NLT / 64, TPW = (kFusedSeamMax + NLW - 1) / NLW, CPL = D / 64;
        const int lw = lt >> 6, ll = lt & 63;
        float sq[TPW][CPL], sk[TPW][CPL], sv[TPW][CPL], sal[TPW], sbe[TPW];
        int swn = 0;
        int lbar = 0;   // loader-barrier target
        auto hrow = [&](int r) { return (lt + NLT * r) / (D / 8); };
        auto hcol = [&](int r, int h) { return h * (D / 2) + 4 * ((lt + NLT * r) % (D / 8)); };
        // the element's slot offset, read once per element by load(): a slot read right before each
        // part's loads would wait (vmcnt) for every load still in flight
        long long so_ld = 0;
        auto load_half = [&](int h) __attribute__((always_inline)) {
            const f4* src = reinterpret_cast<const f4*>(a.T_hat + so_ld * DD);
#pragma unroll
            for (int r = 0; r < TPH; ++r) th[h][r] = src[(hrow(r) * D + hcol(r, h)) / 4];
        };
        auto load_s = [&]() __attribute__((always_inline)) {
            if (!t_role) {  // the transition role needs no S_i
                const f4* srs = reinterpret_cast<const f4*>(a.S + so_ld * DD);
#pragma unroll
                for (int r = 0; r < TPL; ++r) ts[r] = srs[lt + NLT * r];
            }
        };
        // half A comes with the exponent and the seam tokens
        auto load = [&](int el) __attribute__((always_inline)) {
            so_ld = elem(el);
            load_half(0);
            ei = a.T_exp[so_ld];
            if constexpr (SEAM) {
                swn = seg_len(a.seam_tab, el);
                const int bb = chain / a.h_v, hh = chain - (chain / a.h_v) * a.h_v;
                const int hk = (hh * a.h_k) / a.h_v;
#pragma unroll
                for (int m = 0; m < TPW; ++m) {
                    const int t = lw + NLW * m;
                    if (t < swn) {
                        const long long row = (long long)bb * a.n_tokens + seg_start(a.seam_tab, el) + t;
                        const long long qi = (row * a.h_k + hk) * D, vi = (row * a.h_v + hh) * D;
#pragma unroll
                        for (int u = 0; u < CPL; ++u) {
                            const int c = ll + 64 * u;
                            if (a.in_bf16) {
                                sq[m][u] = bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[qi + c]);
                                sk[m][u] = bf16_to_f32(reinterpret_cast<const uint16_t*>(a.k)[qi + c]);
                                sv[m][u] = bf16_to_f32(reinterpret_cast<const uint16_t*>(a.v)[vi + c]);
                            } else {
                                sq[m][u] = reinterpret_cast<const float*>(a.q)[qi + c];
                                sk[m][u] = reinterpret_cast<const float*>(a.k)[qi + c];
                                sv[m][u] = reinterpret_cast<const float*>(a.v)[vi + c];
                            }
                        }
                        sal[m] = a.log_alpha[row * a.h_v + hh];
                        sbe[m] = a.beta[row * a.h_v + hh];
                    }
                }
            }
        };
        auto stage_half = [&](int hh) __attribute__((always_inline)) {
            typedef _Float16 half4 __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int r = 0; r < TPH; ++r) {
                const int row = hrow(r), col = hcol(r, hh);
                const f4 v = th[hh][r];
                half4 h, l;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    h[u] = (_Float16)v[u];
                    l[u] = (_Float16)(v[u] - (float)h[u]);
                }
                *reinterpret_cast<half4*>(&sT[0][row * RS + col]) = h;
                *reinterpret_cast<half4*>(&sT[1][row * RS + col]) = l;
            }
        };
        auto stage_s = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < TPL; ++r) {
                const int f = 4 * (lt + NLT * r);
                *reinterpret_cast<f4*>(&sS[(f / D) * RSS + f % D]) = ts[r];
            }
        };
        // the window's factors, by the loader waves (token t = lw + NLW m belongs to loader wave lw);
        // tokens from w on are zeros in every factor
        auto loader_barrier = [&]() __attribute__((always_inline)) {
            lbar += NLW;
            fold_arrive(sC + 6, lane);
            fold_wait(sC + 6, lbar);
        };
        // sum over the 64 lanes with DPP row sums and four readlanes (no LDS round trips)
        auto wsum = [](float v) {
            v = group_sum<16>(v);
            return (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16))) +
                   (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48)));
        };
        // the window's normalised q rows (fp32) live in the -W' tiles until -W' is formed: rows 0..3 in
        // sWh, 4..7 in sWl, both below their zero row
        auto qrow = [&](int t) __attribute__((always_inline)) {
            return (t < 4 ? reinterpret_cast<float*>(&sWh[0][0]) : reinterpret_cast<float*>(&sWl[0][0])) +
                   (t & 3) * (D + 4);
        };
        auto stage_window = [&]() __attribute__((always_inline)) {
            if constexpr (SEAM) {
            // the window is on the critical path of the next element: issue ahead of the compute waves
            __builtin_amdgcn_s_setprio(2);
            if (lt == 0) sW = swn;
            // 1. each loader wave's tokens: normalised k (fp32 rows, hi/lo K^T) and q (fp32 rows), v rows,
            //    gates
#pragma unroll
            for (int m = 0; m < TPW; ++m) {
                const int t = lw + NLW * m;
                if (t >= WS) continue;
                const bool live = t < swn;   // uniform over the wave
                float fq = 1.f, fk = 1.f;
                if (live && a.qk_l2norm) {
                    float nq = 0.f, nk = 0.f;
#pragma unroll
                    for (int u = 0; u < CPL; ++u) {
                        nq += sq[m][u] * sq[m][u];
                        nk += sk[m][u] * sk[m][u];
                    }
                    nq = wsum(nq);
                    nk = wsum(nk);
                    fq = nq > 0.f ? 1.f / sqrtf(nq) : 0.f;
                    fk = nk > 0.f ? 1.f / sqrtf(nk) : 0.f;
                }
                float* qr = qrow(t);
#pragma unroll
                for (int u = 0; u < CPL; ++u) {
                    const int c = ll + 64 * u;
                    const float kk = live ? sk[m][u] * fk : 0.f;
                    qr[c] = live ? sq[m][u] * fq : 0.f;
                    sKf[t][c] = kk;
                    sVs[t][c] = live ? sv[m][u] : 0.f;
                    const _Float16 kh = (_Float16)kk;
                    sKTh[c][t] = kh;
                    sKTl[c][t] = (_Float16)(kk - (float)kh);
                }
                if (ll == 0) {
                    sGb[t][0] = live ? sal[m] : 0.f;
                    sGb[t][1] = live ? sbe[m] : 0.f;
                }
            }
            loader_barrier();
            // 2a. the 2 w^2 dot products k_t.k_s and q_t.k_s over all loader waves: LPP lanes per product,
            //     32 channels per lane, summed with DPP lane permutations
            auto gsum = [&](float x) {   // G_i of token i: the staged log gates summed in order
                float g = 0.f;
#pragma unroll
                for (int r = 0; r < WS; ++r) g += r <= x ? sGb[r][0] : 0.f;
                return g;
            };
            auto fexp2 = [](float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); };
            {
                constexpr int NPROD = 2 * WS * WS, PPW = NPROD / NLW, LPP = 64 / PPW, CPN = D / LPP;
                static_assert(PPW * NLW == NPROD && LPP * PPW == 64 && (LPP == 2 || LPP == 4), "product split");
                const int pi = PPW * lw + ll / LPP, part = ll % LPP;
                const bool isq = pi >= WS * WS;
                const int pq = isq ? pi - WS * WS : pi, t = pq / WS, s2 = pq % WS;
                const float* x = isq ? qrow(t) : sKf[t];
                const float* y = sKf[s2];
                float acc4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = CPN * part; c < CPN * part + CPN; c += 4) {
                    const float4 a4 = *reinterpret_cast<const float4*>(x + c);
                    const float4 b4 = *reinterpret_cast<const float4*>(y + c);
                    acc4[0] = fmaf(a4.x, b4.x, acc4[0]);
                    acc4[1] = fmaf(a4.y, b4.y, acc4[1]);
                    acc4[2] = fmaf(a4.z, b4.z, acc4[2]);
                    acc4[3] = fmaf(a4.w, b4.w, acc4[3]);
                }
                float dp = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
                dp += dpp_perm<0xb1>(dp);                     // quad_perm [1,0,3,2]
                if constexpr (LPP == 4) dp += dpp_perm<0x4e>(dp);   // quad_perm [2,3,0,1]
                if (part == 0) {
                    const float dec = fexp2(gsum((float)t) - gsum((float)s2));
                    if (isq) {
                        const float mq = (t < swn && s2 <= t) ? dec * dp : 0.f;
                        const _Float16 mh = (_Float16)mq;
                        sMh[t][s2] = mh;
                        sMl[t][s2] = (_Float16)(mq - (float)mh);
                    } else {
                        sLf[t][s2] = (t < swn && s2 < t) ? sGb[t][1] * dec * dp : 0.f;
                    }
                }
            }
            loader_barrier();
            // 2b. wave 0: Tg = (I + L)^-1 diag(beta) by forward substitution (lane j one column); the other
            //     waves: diag(gamma) Q rows; the last wave also Gamma / gamma and Gamma
            if (lw == 0) {
                if (ll < WS) {
                    const int j = ll;
                    float xs[WS];
#pragma unroll
                    for (int i = 0; i < WS; ++i) {
                        float v = i == j ? sGb[j][1] : 0.f;
#pragma unroll
                        for (int s3 = 0; s3 < i; ++s3) v = fmaf(-sLf[i][s3], xs[s3], v);
                        xs[i] = v;
                    }
#pragma unroll
                    for (int i = 0; i < WS; ++i) {
                        const float v = (i < swn && j < swn) ? xs[i] : 0.f;
                        sTgf[i][j] = v;
                        const _Float16 vh = (_Float16)v;
                        sTh[i][j] = vh;
                        sTl[i][j] = (_Float16)(v - (float)vh);
                    }
                }
            } else {
                for (int e = lt - 64; e < WS * D; e += NLT - 64) {
                    const int t = e / D, c = e - (e / D) * D;
                    const float x = t < swn ? fexp2(gsum((float)t)) * qrow(t)[c] : 0.f;
                    const _Float16 xh = (_Float16)x;
                    sQh[t][c] = xh;
                    sQl[t][c] = (_Float16)(x - (float)xh);
                }
                if (lw == NLW - 1 && ll < WS) {
                    const bool live = ll < swn;
                    const float Glast = gsum((float)(swn > 0 ? swn - 1 : 0)), Gl = gsum((float)ll);
                    sGv[ll] = live ? fexp2(Gl) : 0.f;
                    sR[ll] = live ? fexp2(Glast - Gl) : 0.f;
                    if (ll == 0) sGam = swn > 0 ? fexp2(Glast) : 1.f;
                }
            }
            loader_barrier();
            // 3. -Tg diag(gamma) K, hi / lo (over the borrowed q rows, read in phase 2 only)
            for (int e = lt; e < WS * D; e += NLT) {
                const int i = e / D, c = e - (e / D) * D;
                float v = 0.f;
#pragma unroll
                for (int j = 0; j < WS; ++j) v = fmaf(sTgf[i][j] * sGv[j], sKf[j][c], v);
                v = -v;
                const _Float16 vh = (_Float16)v;
                sWh[i][c] = vh;
                sWl[i][c] = (_Float16)(v - (float)vh);
            }
            __builtin_amdgcn_s_setprio(0);
            }
        };
        auto stage = [&]() __attribute__((always_inline)) {
            stage_half(0);
            if (lt == 0) sE = ei;
        };
        if (e0 < e1) {
            load(e0);
            load_half(1);
            load_s();
            if constexpr (SEAM) {
                stage_window();                 // the window of the first element
                fold_arrive(sC + 8, lane);
            }
        }
        // each part of element el goes into LDS once the compute waves are done with that part
        // of element el - 1, and the loads of the same part of el + 1 follow it
        for (int el = e0; el < e1; ++el) {
            const int k = el - e0;
            fold_wait(sC + 3, NB * k);
            stage();                        // T half A, exponent, seam tokens
            fold_arrive(sC + 0, lane);
            if (el + 1 < e1) load(el + 1);
            fold_wait(sC + 4, NB * k);
            stage_half(1);
            fold_arrive(sC + 1, lane);
            if (el + 1 < e1) load_half(1);
            if (!t_role) {
                fold_wait(sC + 5, NB * k);
                stage_s();
                fold_arrive(sC + 2, lane);
                if (el + 1 < e1) load_s();
            }
            if constexpr (SEAM) {
                // the window of el + 1, once the compute waves are done with the window of el (the
                // product of el still runs)
                if (el + 1 < e1) {
                    fold_wait(sC + 7, NB * (k + 1));
                    stage_window();
                    fold_arrive(sC + 8, lane);
                }
            }
        }
        __syncthreads();  // epilogue exponent exchange
        return;
    }

    // ---------------------------------- compute waves ----------------------------------
    const int col0 = 32 * wave;
    floatx16 X[NB];
    if (t_role) {
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
        const _Float16* Th = sT[0];
        const _Float16* Tl = sT[1];
        if (!t_role && a.prefix) {
            {
                float* dst = a.prefix + ((long long)el * a.n_chain + chain) * DD;
#pragma unroll
                for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) dst[(32 * xb + acc_row(half, j)) * D + col0 + l32] = X[xb][j];
            }
        }
        const int kel = el - e0;
        fold_wait(sC + 0, NLW * (kel + 1));   // T half A, exponent and seam tokens of el staged
        if constexpr (SEAM) {
            fold_wait(sC + 8, NLW * (kel + 1));   // the window of el staged
            const int w = sW;
            if (w > 0) {   // uniform
                // an opaque zero keeps the window's per-lane LDS offsets from being hoisted out of the
                // element loop into long-lived registers
                int oz = 0;
                asm volatile("" : "+v"(oz));
                const int wl = lane + oz, l32 = wl & 31, half = wl >> 5;
                const int bb = chain / a.h_v, hh = chain - (chain / a.h_v) * a.h_v;
                // the window's products take X 2^-sx (maximum in [0.5, 1)) as hi/lo f16 operands
                float mx = 0.f;
#pragma unroll
                for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) mx = __builtin_elementwise_maximum(mx, __builtin_fabsf(X[xb][j]));
                const int wx = exp2_of(wave_max(mx));
                const float wsc = ldexpf(1.f, -wx);
                // operands over the window's tokens: lane half h supplies tokens 4h .. 4h + 3 (the
                // other four contraction slots are zero); A rows past the window read the zero row
                auto frag4 = [](const _Float16* p) {
                    const halfx4 x = *reinterpret_cast<const halfx4*>(p);
                    return halfx8{x[0], x[1], x[2], x[3], (_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
                };
                auto split4 = [](const float (&v)[4], halfx8& hi, halfx8& lo) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) hi[i] = lo[i] = (_Float16)0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const _Float16 h = (_Float16)v[i];
                        hi[i] = h;
                        lo[i] = (_Float16)(v[i] - (float)h);
                    }
                };
                auto mma3 = [](halfx8 ah, halfx8 al, halfx8 bh, halfx8 bl, floatx16 c) {
                    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bh, c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bl, c, 0, 0, 0);
                    return __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, c, 0, 0, 0);
                };
                const int rr = l32 < WS ? l32 : WS;
                floatx16 Z = zero16(), O = zero16();
                {
                    // Z = Tg V 2^-wx
                    float vv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) vv[i] = sVs[4 * half + i][col0 + l32] * wsc;
                    halfx8 bh, bl;
                    split4(vv, bh, bl);
                    Z = mma3(frag4(&sTh[rr][4 * half]), frag4(&sTl[rr][4 * half]), bh, bl, Z);
                }
                // Z -= Tg diag(gamma) K X 2^-wx,  O = diag(gamma) Q X 2^-wx; the operand fragments of a
                // step are read one step ahead
                halfx8 fw[2][4];
                auto wload = [&](int ks, halfx8 (&f)[4]) {
                    const int off = 16 * ks + 4 * half;
                    f[0] = t_frag(&sWh[rr][off]);
                    f[1] = t_frag(&sWl[rr][off]);
                    f[2] = t_frag(&sQh[rr][off]);
                    f[3] = t_frag(&sQl[rr][off]);
                };
                wload(0, fw[0]);
#pragma unroll
                for (int ks = 0; ks < 2 * NB; ++ks) {
                    if (ks + 1 < 2 * NB) wload(ks + 1, fw[(ks + 1) & 1]);
                    halfx8 bh, bl;
                    split_hilo(X[ks >> 1], ks & 1, wsc, bh, bl);
                    const halfx8(&f)[4] = fw[ks & 1];
                    Z = mma3(f[0], f[1], bh, bl, Z);
                    O = mma3(f[2], f[3], bh, bl, O);
                    __builtin_amdgcn_sched_barrier(0);
                }
                {
                    // O += Mq Z
                    const float zz[4] = {Z[0], Z[1], Z[2], Z[3]};
                    halfx8 bh, bl;
                    split4(zz, bh, bl);
                    O = mma3(frag4(&sMh[rr][4 * half]), frag4(&sMl[rr][4 * half]), bh, bl, O);
                }
                if (a.o) {
                    // o_t for the window tokens t = 4h + j of this lane's column
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int t = 4 * half + j;
                        if (t < w) {
                            const float ov = ldexpf(O[j], wx);
                            const long long row = (long long)bb * a.n_tokens + seg_start(a.seam_tab, el) + t;
                            const long long oi = (row * a.h_v + hh) * D + col0 + l32;
                            if (a.out_bf16) reinterpret_cast<uint16_t*>(a.o)[oi] = f32_to_bf16(ov);
                            else reinterpret_cast<float*>(a.o)[oi] = ov;
                        }
                    }
                }
                {
                    // S <- Gamma S + K^T diag(Gamma / gamma) Z
                    float vn[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) vn[j] = ldexpf(Z[j], wx) * sR[4 * half + j];
                    halfx8 bh, bl;
                    split4(vn, bh, bl);
                    const float Gm = sGam;
#pragma unroll
                    for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
                        for (int j = 0; j < 16; ++j) X[rt][j] *= Gm;
                        X[rt] = mma3(frag4(&sKTh[32 * rt + l32][4 * half]), frag4(&sKTl[32 * rt + l32][4 * half]), bh,
                                     bl, X[rt]);
                    }
                }
            }
            fold_arrive(sC + 7, lane);   // the window of el consumed
        }
        const int ecur = sE;
        // scale this wave's columns to max |x| in [0.5, 1) before the hi/lo split
        float m = 0.f;
#pragma unroll
        for (int xb = 0; xb < NB; ++xb)
#pragma unroll
            for (int j = 0; j < 16; ++j) m = __builtin_elementwise_maximum(m, __builtin_fabsf(X[xb][j]));
        const int sx = exp2_of(wave_max(m));
        const float sc = ldexpf(1.f, -sx);
        floatx16 acc[NB];
#pragma unroll
        for (int ob = 0; ob < NB; ++ob) acc[ob] = zero16();
        // steps (kb, st, ob); the T_i fragments (hi, lo) of a step are read LA steps ahead
        // (a ring of LA + 1) so that LDS latency hides behind the products of earlier steps
        constexpr int NSTEP = NB * 2 * NB, LA = 1, NR = LA + 1;
        auto tload = [&](int i, halfx8& ah, halfx8& al) {
            const int ob = i % NB, ks = i / NB;  // ks = 2 kb + st
            const int off = (32 * ob + l32) * RS + 16 * ks + 4 * half;
            ah = t_frag(Th + off);
            al = t_frag(Tl + off);
        };
        halfx8 fh[NR], fl[NR], bh, bl;
#pragma unroll
        for (int i = 0; i < LA; ++i) tload(i, fh[i], fl[i]);
#pragma unroll
        for (int i = 0; i < NSTEP; ++i) {
            // steps NSTEP / 2 .. read T half B (contraction indices D / 2 ..)
            if (i + LA == NSTEP / 2) fold_wait(sC + 1, NLW * (kel + 1));
            if (i + LA < NSTEP) tload(i + LA, fh[(i + LA) % NR], fl[(i + LA) % NR]);
            const int ob = i % NB, ks = i / NB;
            if (ob == 0) split_hilo(X[ks >> 1], ks & 1, sc, bh, bl);
            acc[ob] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fl[i % NR], bh, acc[ob], 0, 0, 0);
            acc[ob] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fh[i % NR], bl, acc[ob], 0, 0, 0);
            acc[ob] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fh[i % NR], bh, acc[ob], 0, 0, 0);
            if (i == NSTEP / 2 - 1) fold_arrive(sC + 3, lane);   // every half-A fragment read
            __builtin_amdgcn_sched_barrier(0);
        }
        fold_arrive(sC + 4, lane);   // every half-B fragment read
        if (t_role) {
            // X = T_i (X 2^-sx): exponent += sx + e_i, then renormalise
            float mm = 0.f;
#pragma unroll
            for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                for (int j = 0; j < 16; ++j) mm = __builtin_elementwise_maximum(mm, __builtin_fabsf(acc[xb][j]));
            const int e = exp2_of(wave_max(mm));
            const float r = ldexpf(1.f, -e);
#pragma unroll
            for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                for (int j = 0; j < 16; ++j) X[xb][j] = acc[xb][j] * r;
            ew += sx + ecur + e;
        } else {
            fold_wait(sC + 2, NLW * (kel + 1));   // S_el staged
#pragma unroll
            for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    X[xb][j] = ldexpf(acc[xb][j], sx + ecur) + sS[(32 * xb + acc_row(half, j)) * RSS + col0 + l32];
            fold_arrive(sC + 5, lane);
        }
    }

    if (t_role && lane == 0) sEw[wave] = ew;
    __syncthreads();  // epilogue exponent exchange
    if (t_role) {
        int emax = sEw[0];
        for (int w = 1; w < NB; ++w) emax = max(emax, sEw[w]);
        float* dst = a.out_T + ((long long)blk * a.n_chain + chain) * DD;
#pragma unroll
        for (int xb = 0; xb < NB; ++xb)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                dst[(32 * xb + acc_row(half, j)) * D + col0 + l32] = ldexpf(X[xb][j], ew - emax);
        if (tid == 0) a.out_e[(long long)blk * a.n_chain + chain] = emax;
    } else if (a.out_S) {
        float* dst = a.out_S + ((long long)blk * a.n_chain + chain) * DD;
#pragma unroll
        for (int xb = 0; xb < NB; ++xb)
#pragma unroll
            for (int j = 0; j < 16; ++j) dst[(32 * xb + acc_row(half, j)) * D + col0 + l32] = X[xb][j];
    }
}

// Diagonal (T a d_k vector) and scalar (T one value) kinds: elementwise.  Entry (r, c) of the
// state only ever meets T[r] (or the scalar T), so a chain's d x d state is split over NZ
// workgroups of contiguous rows, each reading the T entries of its own rows directly (no LDS
// exchange, no barrier on the state path).  The slice-0 workgroup also carries the running
// product of the transitions, renormalised by its maximum after every element.
template <int D>
constexpr int fold_diag_slices() { return D * D / (256 * 4); }

template <int D>
__global__ __launch_bounds__(256) void fold_diag_kernel(FoldArgs a) {
    constexpr int NT = 256;
    constexpr int PER = 4;                      // state entries per thread
    constexpr int NZ = fold_diag_slices<D>();   // row slices per chain
    constexpr int SL = D * D / NZ;              // entries per slice
    static_assert(NZ * NT * PER == D * D && SL % D == 0, "slices of whole rows");
    __shared__ float sRed[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int chain = blockIdx.x, blk = blockIdx.y, z = blockIdx.z;
    const bool scalar = a.kind == 2;
    const bool carry_T = a.out_T && z == 0;
    const int e0 = blk * a.per_block;
    const int e1 = min(a.n_elem, e0 + a.per_block);
    const long long DD = (long long)D * D;
    const int tlen = scalar ? 1 : D;
    const int base = z * SL;
    int trow[PER];  // T index of each entry's row
#pragma unroll
    for (int r = 0; r < PER; ++r) trow[r] = scalar ? 0 : (base + tid + NT * r) / D;

    float x[PER];
    if (a.init_S) {
        const float* src = a.init_S + ((long long)blk * a.n_chain + chain) * DD + base;
#pragma unroll
        for (int r = 0; r < PER; ++r) x[r] = src[tid + NT * r];
    } else {
#pragma unroll
        for (int r = 0; r < PER; ++r) x[r] = 0.f;
    }
    float tv = 1.f;  // slice 0: thread tid < tlen owns T[tid]
    int te = 0;
    for (int el = e0; el < e1; ++el) {
        const int slot = a.slot ? a.slot[el] : el;
        const long long so = (long long)slot * a.n_chain + chain;
        if (a.prefix) {
            float* dst = a.prefix + ((long long)el * a.n_chain + chain) * DD + base;
#pragma unroll
            for (int r = 0; r < PER; ++r) dst[tid + NT * r] = x[r];
        }
        const float* Si = a.S + so * DD + base;
        if (a.naive) {
#pragma unroll
            for (int r = 0; r < PER; ++r) x[r] += Si[tid + NT * r];
            continue;
        }
        const float* Ti = a.T_hat + so * tlen;
        const int ei = a.T_exp[so];
#pragma unroll
        for (int r = 0; r < PER; ++r) x[r] = ldexpf(Ti[trow[r]] * x[r], ei) + Si[tid + NT * r];
        if (carry_T) {
            // running product of transitions, renormalised by the block max
            if (tid < tlen) tv *= Ti[tid];
            float m = tid < tlen ? fabsf(tv) : 0.f;
            m = wave_max(m);
            if (lane == 0) sRed[wave] = m;
            __syncthreads();
            const float mm = fmaxf(fmaxf(sRed[0], sRed[1]), fmaxf(sRed[2], sRed[3]));
            const int e = exp2_of(mm);
            tv = ldexpf(tv, -e);
            te += ei + e;
            __syncthreads();
        }
    }
    if (a.out_S) {
        float* dst = a.out_S + ((long long)blk * a.n_chain + chain) * DD + base;
#pragma unroll
        for (int r = 0; r < PER; ++r) dst[tid + NT * r] = x[r];
    }
    if (carry_T) {
        if (tid < tlen) a.out_T[((long long)blk * a.n_chain + chain) * tlen + tid] = tv;
        if (tid == 0) a.out_e[(long long)blk * a.n_chain + chain] = te;
    }
}

// Dense kind, running state only (no composed transition, no seam window).  Under
// S <- T_i S + S_i the columns of a chain's state never mix, so a chain's d columns are split
// into d/16 parts of one workgroup each, and the part's rows into four compute waves (d/4 rows
// each, 16-row tiles).  A step forms T_i X for the part with 16x16x32 f16 products on hi/lo
// splits of both operands (three products per pair, the lo x lo term dropped): T_i is staged
// row-major in LDS as hi/lo f16 by the loader waves (double buffered; the loads run two
// elements ahead of use), the part's columns go through LDS transposed, as hi/lo f16 after a
// per-column scaling by an exact power of two that the four waves agree on through LDS
// (every column's maximum |x| lands in [0.5, 1)).  S_i is added in fp32 as read from HBM.
// The workgroups of one chain are dealt to the same XCD, so T_i comes from HBM once and from
// that XCD's L2 for the other parts.
template <int D>
constexpr int split_loader_waves() { return D == 128 ? 8 : 4; }

template <int D>
__global__ __launch_bounds__((4 + split_loader_waves<D>()) * 64) void fold_split_kernel(FoldArgs a) {
    constexpr int NCW = 4;                       // compute waves
    constexpr int NLW = split_loader_waves<D>(); // loader waves
    constexpr int NLT = NLW * 64;
    constexpr int NCP = D / 16;                  // column parts per chain
    constexpr int RPW = D / NCW;                 // rows per compute wave
    constexpr int NT = RPW / 16;                 // 16-row tiles per compute wave
    constexpr int KS = D / 32;                   // 32-deep contraction steps
    constexpr int RS = D + 8;                    // LDS row stride (halves)
    constexpr int TPL = D * D / (4 * NLT);       // float4 of T_i per loader thread
    static_assert(TPL * 4 * NLT == D * D && NT * 16 == RPW, "split");
    __shared__ __align__(16) _Float16 sT[2][2][D * RS];   // [buffer][hi, lo], row-major
    __shared__ __align__(16) _Float16 sX[2][16 * RS];     // [hi, lo][column][row]
    __shared__ __align__(16) float sM[16][NCW * 4];       // [column][wave, lane group] partial maxima
    // counters: T consumed (one arrival per compute wave and element), column maxima written,
    // columns written (one per compute wave and step), T staged into buffer 0 and into buffer 1
    // (one per loader wave and element).  The staged counts are kept per buffer: before its
    // first wait for a consumed element a loader wave may stage elements 0 and 1 while another
    // has not yet staged element 0, so one count over both buffers could reach a target early
    __shared__ int sC[5];

    // workgroup -> (chain, part): ids congruent mod 8 share an XCD
    const int id = blockIdx.x, r8 = id >> 3;
    const int cp = r8 % NCP;
    const int chain = (r8 / NCP) * 8 + (id & 7);
    if (chain >= a.n_chain) return;   // padding of the grid to whole groups of 8 chains
    const int blk = blockIdx.y;
    const int e0 = blk * a.per_block;
    const int ne = max(0, min(a.n_elem, e0 + a.per_block) - e0);
    const long long DD = (long long)D * D;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (tid < 5) sC[tid] = 0;
    __syncthreads();

    // slots of the elements in batches of 64 (lane i: element b0 + i), one vector load per batch,
    // so that no per-element slot read has to wait (vmcnt) for the loads in flight
    int sl_b = 0, eb = -1;
    auto slot_batch = [&](int k) __attribute__((always_inline)) {
        const int b0 = k & ~63;
        if (b0 != eb) {
            eb = b0;
            const int kk = b0 + lane;
            sl_b = kk < ne ? (a.slot ? a.slot[e0 + kk] : e0 + kk) : 0;
        }
        return b0;
    };

    if (wave >= NCW) {
        // ============================ loader waves ============================
        typedef float f4 __attribute__((ext_vector_type(4)));
        typedef _Float16 half4 __attribute__((ext_vector_type(4)));
        const int lt = tid - NCW * 64;
        f4 tr[2][TPL];
        auto load = [&](int k, f4 (&dst)[TPL]) __attribute__((always_inline)) {
            const int b0 = slot_batch(k);
            const int sl = __builtin_amdgcn_readlane(sl_b, k - b0);
            const f4* src = reinterpret_cast<const f4*>(a.T_hat + ((long long)sl * a.n_chain + chain) * DD);
#pragma unroll
            for (int r = 0; r < TPL; ++r) dst[r] = src[lt + NLT * r];
        };
        auto stage = [&](const f4 (&src)[TPL], int buf) __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < TPL; ++r) {
                const int f = lt + NLT * r, row = f / (D / 4), c = 4 * (f % (D / 4));
                half4 h, l;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    h[u] = (_Float16)src[r][u];
                    l[u] = (_Float16)(src[r][u] - (float)h[u]);
                }
                *reinterpret_cast<half4*>(&sT[buf][0][row * RS + c]) = h;
                *reinterpret_cast<half4*>(&sT[buf][1][row * RS + c]) = l;
            }
        };
        if (ne > 0) load(0, tr[0]);
        if (ne > 1) load(1, tr[1]);
        auto body = [&](auto bc, int k) __attribute__((always_inline)) {
            constexpr int B = decltype(bc)::value;   // register set and LDS buffer of element k
            if (k >= 2) fold_wait(sC + 0, NCW * (k - 1));   // element k - 2 (same buffer) consumed
            stage(tr[B], B);
            fold_arrive(sC + 3 + B, lane);
            if (k + 2 < ne) load(k + 2, tr[B]);
        };
        for (int k = 0; k < ne; k += 2) {
            body(std::integral_constant<int, 0>{}, k);
            if (k + 1 < ne) body(std::integral_constant<int, 1>{}, k + 1);
        }
        return;
    }

    // ============================ compute waves ============================
    typedef _Float16 half4 __attribute__((ext_vector_type(4)));
    const int w = wave, g = lane >> 4, cl = lane & 15;
    const int col = 16 * cp + cl;
    const int rbase = RPW * w + 4 * g;   // row of tile t, register j: rbase + 16 t + j
    floatx4 X[NT];
    if (a.init_S) {
        const float* src = a.init_S + ((long long)blk * a.n_chain + chain) * DD + col;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) X[t][j] = src[(rbase + 16 * t + j) * D];
    } else {
#pragma unroll
        for (int t = 0; t < NT; ++t) X[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    // exponents of the batch's elements (lane i: element b0 + i)
    int ex_b = 0, ebx = -1;
    floatx4 sr[2][NT];   // S_i of elements k and k + 1, read two elements ahead
    auto load_s = [&](int k, floatx4 (&dst)[NT]) __attribute__((always_inline)) {
        const int b0 = slot_batch(k);
        const int sl = __builtin_amdgcn_readlane(sl_b, k - b0);
        const float* src = a.S + ((long long)sl * a.n_chain + chain) * DD + col;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[t][j] = src[(rbase + 16 * t + j) * D];
    };
    auto exponent = [&](int k) __attribute__((always_inline)) {
        const int b0 = k & ~63;
        if (b0 != ebx) {
            ebx = b0;
            slot_batch(k);
            ex_b = b0 + lane < ne ? a.T_exp[(long long)sl_b * a.n_chain + chain] : 0;
        }
        return __builtin_amdgcn_readlane(ex_b, k - b0);
    };
    if (ne > 0) load_s(0, sr[0]);
    if (ne > 1) load_s(1, sr[1]);
    auto body = [&](auto bc, int k) __attribute__((always_inline)) {
        constexpr int B = decltype(bc)::value;
        const int el = e0 + k;
        // 1. the columns' maxima over the four waves
        float m = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) m = __builtin_elementwise_maximum(m, __builtin_fabsf(X[t][j]));
        sM[cl][4 * w + g] = m;
        fold_arrive(sC + 1, lane);
        fold_wait(sC + 1, NCW * (k + 1));
        {
            const float4* mv = reinterpret_cast<const float4*>(&sM[cl][0]);
            float mm = 0.f;
#pragma unroll
            for (int q = 0; q < NCW; ++q) {
                const float4 v = mv[q];
                mm = __builtin_elementwise_maximum(
                    mm, __builtin_elementwise_maximum(__builtin_elementwise_maximum(v.x, v.y),
                                                      __builtin_elementwise_maximum(v.z, v.w)));
            }
            m = mm;
        }
        const int sx = exp2_of(m);
        // 2. the columns as hi/lo f16, scaled by 2^-sx, transposed into LDS
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            half4 h, l;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v = ldexpf(X[t][j], -sx);
                h[j] = (_Float16)v;
                l[j] = (_Float16)(v - (float)h[j]);
            }
            *reinterpret_cast<half4*>(&sX[0][cl * RS + rbase + 16 * t]) = h;
            *reinterpret_cast<half4*>(&sX[1][cl * RS + rbase + 16 * t]) = l;
        }
        fold_arrive(sC + 2, lane);
        // the T_el fragments of this wave's rows, read while the other waves write their columns
        fold_wait(sC + 3 + B, NLW * (k / 2 + 1));   // T_el staged in buffer B
        const _Float16* Th = &sT[B][0][0];
        const _Float16* Tl = &sT[B][1][0];
        halfx8 fah[KS][NT], fal[KS][NT];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int ao = (RPW * w + 16 * t + cl) * RS + 32 * ks + 8 * g;
                fah[ks][t] = *reinterpret_cast<const halfx8*>(Th + ao);
                fal[ks][t] = *reinterpret_cast<const halfx8*>(Tl + ao);
            }
        if (a.prefix) {
            float* dst = a.prefix + ((long long)el * a.n_chain + chain) * DD + col;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) dst[(rbase + 16 * t + j) * D] = X[t][j];
        }
        const int ecur = exponent(k);
        fold_wait(sC + 2, NCW * (k + 1));
        // 3. T_el X: rows of this wave, the part's 16 columns; the cross terms and the main term
        // in separate accumulators (four independent product chains)
        floatx4 acc[NT], acs[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = acs[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int kof = 32 * ks + 8 * g;
            const halfx8 bh = *reinterpret_cast<const halfx8*>(&sX[0][cl * RS + kof]);
            const halfx8 bl = *reinterpret_cast<const halfx8*>(&sX[1][cl * RS + kof]);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                acs[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fal[ks][t], bh, acs[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fah[ks][t], bh, acc[t], 0, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) acs[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fah[ks][t], bl, acs[t], 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] += acs[t];
        fold_arrive(sC + 0, lane);   // buffer B and the columns read
        // 4. S <- 2^(e + sx) (T_el X 2^-sx) + S_el
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) X[t][j] = ldexpf(acc[t][j], ecur + sx) + sr[B][t][j];
        if (k + 2 < ne) load_s(k + 2, sr[B]);
    };
    for (int k = 0; k < ne; k += 2) {
        body(std::integral_constant<int, 0>{}, k);
        if (k + 1 < ne) body(std::integral_constant<int, 1>{}, k + 1);
    }
    if (a.out_S) {
        float* dst = a.out_S + ((long long)blk * a.n_chain + chain) * DD + col;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[(rbase + 16 * t + j) * D] = X[t][j];
    }
}

hipError_t launch_fold_split(const FoldArgs& a, int d, hipStream_t s) {
    if (a.kind != 0 || a.naive || a.seam || a.out_T) return hipErrorInvalidValue;
    const dim3 grid(((a.n_chain + 7) / 8) * 8 * (d / 16), a.n_block);
    if (d == 128)
        hipLaunchKernelGGL((fold_split_kernel<128>), grid, dim3((4 + split_loader_waves<128>()) * 64), 0, s, a);
    else if (d == 64)
        hipLaunchKernelGGL((fold_split_kernel<64>), grid, dim3((4 + split_loader_waves<64>()) * 64), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_fold(const FoldArgs& a, int d, int with_T, hipStream_t s) {
    if (a.kind == 0 && !a.naive) {
        // role 1 (the composed transition) only when its outputs are wanted
        const dim3 g3(a.n_chain, a.n_block, (with_T && a.out_T) ? 2 : 1);
        if (a.seam) {
            // the fused warm path: one block per chain, S only
            if (a.n_block != 1 || with_T) return hipErrorInvalidValue;
            if (d == 128) hipLaunchKernelGGL((fold_dense_kernel<128, true>), g3, dim3(768), 0, s, a);
            else if (d == 64) hipLaunchKernelGGL((fold_dense_kernel<64, true>), g3, dim3(384), 0, s, a);
            else return hipErrorInvalidValue;
        } else if (d == 128) hipLaunchKernelGGL((fold_dense_kernel<128, false>), g3, dim3(768), 0, s, a);
        else if (d == 64) hipLaunchKernelGGL((fold_dense_kernel<64, false>), g3, dim3(384), 0, s, a);
        else return hipErrorInvalidValue;
    } else {
        // naive addition of any kind, and the diagonal / scalar kinds
        if (d == 128)
            hipLaunchKernelGGL((fold_diag_kernel<128>), dim3(a.n_chain, a.n_block, fold_diag_slices<128>()), dim3(256), 0, s, a);
        else if (d == 64)
            hipLaunchKernelGGL((fold_diag_kernel<64>), dim3(a.n_chain, a.n_block, fold_diag_slices<64>()), dim3(256), 0, s, a);
        else return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace hypic
