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
// previous element (LDS counters, no workgroup barrier per element).
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
// (q, k, v rows, gates) and stages it in LDS (float32, q and k L2-normalised on request);
// before each element's product the compute waves run the gated delta rule over those tokens
// on their accumulator-resident columns: u = k^T S (lane-local partial over its 64 rows plus
// the other lane half's), S <- alpha (S - beta k u^T) + beta k v^T, o = S^T q.
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
    __shared__ __align__(16) float sQk[WS][2][D];   // seam q, k rows
    __shared__ __align__(16) float sVs[WS][D];      // seam v rows
    __shared__ float sGb[WS][2];                    // alpha, beta
    __shared__ int sW;                              // seam tokens of the staged element
    // hand-off counters: T_i column half A, half B and S_i staged (one arrival per loader wave),
    // then consumed (one per compute wave)
    __shared__ int sC[6];

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
    if (tid < 6) sC[tid] = 0;
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
        auto hrow = [&](int r) { return (lt + NLT * r) / (D / 8); };
        auto hcol = [&](int r, int h) { return h * (D / 2) + 4 * ((lt + NLT * r) % (D / 8)); };
        auto load_half = [&](int el, int h) __attribute__((always_inline)) {
            const f4* src = reinterpret_cast<const f4*>(a.T_hat + elem(el) * DD);
#pragma unroll
            for (int r = 0; r < TPH; ++r) th[h][r] = src[(hrow(r) * D + hcol(r, h)) / 4];
        };
        auto load_s = [&](int el) __attribute__((always_inline)) {
            if (!t_role) {  // the transition role needs no S_i
                const f4* srs = reinterpret_cast<const f4*>(a.S + elem(el) * DD);
#pragma unroll
                for (int r = 0; r < TPL; ++r) ts[r] = srs[lt + NLT * r];
            }
        };
        // half A comes with the exponent and the seam tokens
        auto load = [&](int el) __attribute__((always_inline)) {
            const long long so = elem(el);
            load_half(el, 0);
            ei = a.T_exp[so];
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
                        sal[m] = expf(a.log_alpha[row * a.h_v + hh]);
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
        auto stage = [&]() __attribute__((always_inline)) {
            stage_half(0);
            if (lt == 0) sE = ei;
            if constexpr (SEAM) {
                if (lt == 0) sW = swn;
#pragma unroll
                for (int m = 0; m < TPW; ++m) {
                    const int t = lw + NLW * m;
                    if (t < swn) {   // uniform over the wave
                        float fq = 1.f, fk = 1.f;
                        if (a.qk_l2norm) {
                            float nq = 0.f, nk = 0.f;
#pragma unroll
                            for (int u = 0; u < CPL; ++u) {
                                nq += sq[m][u] * sq[m][u];
                                nk += sk[m][u] * sk[m][u];
                            }
                            nq = wave_sum(nq);
                            nk = wave_sum(nk);
                            fq = nq > 0.f ? 1.f / sqrtf(nq) : 0.f;
                            fk = nk > 0.f ? 1.f / sqrtf(nk) : 0.f;
                        }
#pragma unroll
                        for (int u = 0; u < CPL; ++u) {
                            sQk[t][0][ll + 64 * u] = sq[m][u] * fq;
                            sQk[t][1][ll + 64 * u] = sk[m][u] * fk;
                            sVs[t][ll + 64 * u] = sv[m][u];
                        }
                        if (ll == 0) {
                            sGb[t][0] = sal[m];
                            sGb[t][1] = sbe[m];
                        }
                    }
                }
            }
        };
        if (e0 < e1) {
            load(e0);
            load_half(e0, 1);
            load_s(e0);
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
            if (el + 1 < e1) load_half(el + 1, 1);
            if (!t_role) {
                fold_wait(sC + 5, NB * k);
                stage_s();
                fold_arrive(sC + 2, lane);
                if (el + 1 < e1) load_s(el + 1);
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
            const int w = sW;
            const int bb = chain / a.h_v, hh = chain - (chain / a.h_v) * a.h_v;
            for (int t = 0; t < w; ++t) {
                const float* kr = sQk[t][1];
                const float* qr = sQk[t][0];
                // u = k^T S for this lane's column: its 64 rows, then the other half's
                float up[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const floatx4 k4 = *reinterpret_cast<const floatx4*>(kr + 32 * xb + 8 * g + 4 * half);
#pragma unroll
                        for (int i = 0; i < 4; ++i) up[i] = fmaf(k4[i], X[xb][4 * g + i], up[i]);
                    }
                float u = (up[0] + up[1]) + (up[2] + up[3]);
                u += __shfl_xor(u, 32, 64);
                const float al = sGb[t][0], be = sGb[t][1];
                // S <- al (S - be k u) + be k v  =  al S + k (be (v - al u))
                const float cf = be * (sVs[t][col0 + l32] - al * u);
                float op[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const floatx4 k4 = *reinterpret_cast<const floatx4*>(kr + 32 * xb + 8 * g + 4 * half);
                        const floatx4 q4 = *reinterpret_cast<const floatx4*>(qr + 32 * xb + 8 * g + 4 * half);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float x = fmaf(k4[i], cf, al * X[xb][4 * g + i]);
                            X[xb][4 * g + i] = x;
                            op[i] = fmaf(q4[i], x, op[i]);
                        }
                    }
                float ov = (op[0] + op[1]) + (op[2] + op[3]);
                ov += __shfl_xor(ov, 32, 64);
                if (half == 0 && a.o) {
                    const long long row = (long long)bb * a.n_tokens + seg_start(a.seam_tab, el) + t;
                    const long long oi = (row * a.h_v + hh) * D + col0 + l32;
                    if (a.out_bf16) reinterpret_cast<uint16_t*>(a.o)[oi] = f32_to_bf16(ov);
                    else reinterpret_cast<float*>(a.o)[oi] = ov;
                }
            }
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
